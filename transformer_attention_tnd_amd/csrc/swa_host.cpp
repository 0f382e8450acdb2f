// Host side of the library: argument validation, the varlen tile schedule and
// the C ABI entry points declared in include/swa.h.
//
// The tile schedule is the host half of skipping masked work: the actual_seq
// values drive the tiling (aclnnFlashAttentionUnpaddingScoreGradV2 explainer,
// section 8.1, where the actual_seq inputs are value-dependent), and with
// sparse_mode 4 every tile outside the band -pre_tokens <= j - i <= next_tokens
// is never visited (op-plugin sliding-window blog, section 1.3).  The causal
// modes 2 (LEFT_UP_CAUSAL) and 3 (RIGHT_DOWN_CAUSAL) of the same section are
// bands too: j <= i, and j - i <= Skv - Sq (the diagonal from the top-left or
// the bottom-right corner), so every mode reaches the kernels as a band per
// sequence.

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/swa.h"
#include "swa_internal.hpp"

namespace swa {
namespace {

thread_local std::string g_err;

swa_status fail(swa_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

struct Seq {
  int64_t q0, sq, k0, skv;
  int32_t b;
  int64_t drop_base;  // first dropout-mask bit of this sequence (sum of N Sq Skv before it)
};

int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return q;
}
int64_t ceil_div(int64_t a, int64_t b) { return -floor_div(-a, b); }

// The mask of one sequence as a band: key j is allowed for query i iff
// -pre <= j - i <= next (sequence-local indices); on == false: no mask.
struct Band {
  bool on;
  int64_t pre, next;
};
constexpr int64_t kWide = int64_t(1) << 40;  // wider than any sequence

constexpr int64_t kMaxT = int64_t(1) << 20;  // explainer 6.3: T in 1..1M

swa_status check_sizes(int64_t num_seqs, int64_t t_q, int64_t t_kv, int64_t num_heads,
                       int64_t head_dim, int32_t dtype) {
  if (num_seqs < 1 || num_seqs > 2048)
    return fail(SWA_ERR_INVALID, "num_seqs must be in 1..2048, got " + std::to_string(num_seqs));
  if (t_q < 1 || t_q > kMaxT || t_kv < 1 || t_kv > kMaxT)
    return fail(SWA_ERR_INVALID, "t_q and t_kv must be in 1..1048576, got " +
                                     std::to_string(t_q) + ", " + std::to_string(t_kv));
  if (num_heads < 1 || num_heads > 256)
    return fail(SWA_ERR_INVALID, "num_heads must be in 1..256, got " + std::to_string(num_heads));
  if (head_dim < 1 || head_dim > 768)
    return fail(SWA_ERR_INVALID, "head_dim must be in 1..768, got " + std::to_string(head_dim));
  if (dtype != SWA_DTYPE_FP32 && dtype != SWA_DTYPE_BF16 && dtype != SWA_DTYPE_FP16)
    return fail(SWA_ERR_INVALID, "dtype must be 0 (fp32), 1 (bf16) or 2 (fp16), got " +
                                     std::to_string(dtype));
  if (dtype == SWA_DTYPE_FP16)
    return fail(SWA_ERR_UNSUPPORTED, "fp16 inputs are not supported (fp32 and bf16 are)");
  if (head_dim != 64 && head_dim != 128)
    return fail(SWA_ERR_UNSUPPORTED,
                "head_dim " + std::to_string(head_dim) + " is not supported (64 and 128 are)");
  return SWA_OK;
}

// Parse the cumulative ends into participating sequences.
swa_status parse_seqs(const Problem& p, std::vector<Seq>& seqs, int64_t* end_q,
                      int64_t* end_kv) {
  seqs.clear();
  int64_t prev_q = 0, prev_kv = 0;
  bool trail_q = false, trail_kv = false;
  for (int64_t b = 0; b < p.num_seqs; ++b) {
    const int64_t cq = p.cu_q[b], ck = p.cu_kv[b];
    if (cq < 0 || ck < 0) return fail(SWA_ERR_INVALID, "cu_seqlens entries must be >= 0");
    if (trail_q || trail_kv) {
      if (cq != 0 || ck != 0)
        return fail(SWA_ERR_INVALID, "cu_seqlens: nonzero entry after the trailing zero run at "
                                     "batch " + std::to_string(b));
      continue;
    }
    const bool tq = (cq == 0 && prev_q > 0), tk = (ck == 0 && prev_kv > 0);
    if (tq != tk)
      return fail(SWA_ERR_INVALID, "cu_seqlens_q and cu_seqlens_kv disagree on which batches "
                                   "participate (batch " + std::to_string(b) + ")");
    if (tq) {
      trail_q = trail_kv = true;
      continue;
    }
    if (cq < prev_q || ck < prev_kv)
      return fail(SWA_ERR_INVALID, "cu_seqlens must be non-decreasing (batch " +
                                       std::to_string(b) + ")");
    const int64_t base = seqs.empty() ? 0
                                      : seqs.back().drop_base +
                                            p.num_heads * seqs.back().sq * seqs.back().skv;
    seqs.push_back(Seq{prev_q, cq - prev_q, prev_kv, ck - prev_kv, static_cast<int32_t>(b), base});
    prev_q = cq;
    prev_kv = ck;
  }
  if (prev_q > p.t_q)
    return fail(SWA_ERR_INVALID, "last cu_seqlens_q end " + std::to_string(prev_q) +
                                     " exceeds t_q " + std::to_string(p.t_q));
  if (prev_kv > p.t_kv)
    return fail(SWA_ERR_INVALID, "last cu_seqlens_kv end " + std::to_string(prev_kv) +
                                     " exceeds t_kv " + std::to_string(p.t_kv));
  if (p.sparse_mode == 4) {
    for (const Seq& s : seqs)
      if (s.sq != s.skv)
        return fail(SWA_ERR_UNSUPPORTED,
                    "sparse_mode 4 needs equal query and key lengths per batch; batch " +
                        std::to_string(s.b) + " has " + std::to_string(s.sq) + " and " +
                        std::to_string(s.skv));
  }
  if (p.drop_mask) {  // the mask covers sum_b N Sq Skv bits, read as whole 32-bit words
    int64_t bits = 0;
    for (const Seq& s : seqs) bits += p.num_heads * s.sq * s.skv;
    const int64_t need = (bits + 31) / 32 * 4;
    if (static_cast<int64_t>(p.drop_mask_bytes) < need)
      return fail(SWA_ERR_INVALID, "drop_mask has " + std::to_string(p.drop_mask_bytes) +
                                       " bytes, needs " + std::to_string(need) +
                                       " (the mask bits rounded up to whole 32-bit words)");
  }
  *end_q = prev_q;
  *end_kv = prev_kv;
  return SWA_OK;
}

swa_status validate(const Problem& p, std::vector<Seq>& seqs, int64_t* end_q, int64_t* end_kv) {
  if (!p.cu_q || !p.cu_kv) return fail(SWA_ERR_NULLPTR, "cu_seqlens_q / cu_seqlens_kv is NULL");
  swa_status s = check_sizes(p.num_seqs, p.t_q, p.t_kv, p.num_heads, p.head_dim, p.dtype);
  if (s != SWA_OK) return s;
  // dropout with a given mask (API doc, dropMaskOptional / keepProbOptional; explainer 6.3)
  if (p.drop_mask) {
    if (!std::isfinite(p.keep_prob) || !(p.keep_prob > 0.0 && p.keep_prob <= 1.0))
      return fail(SWA_ERR_INVALID, "keep_prob must be in (0, 1], got " + std::to_string(p.keep_prob));
    if (reinterpret_cast<uintptr_t>(p.drop_mask) % 4 != 0)
      return fail(SWA_ERR_INVALID, "drop_mask must be 4-byte aligned");
  }
  // explainer 6.2: the query head count is a whole multiple of the key/value head count
  if (p.num_kv_heads < 1 || p.num_kv_heads > p.num_heads || p.num_heads % p.num_kv_heads != 0)
    return fail(SWA_ERR_INVALID, "num_heads (" + std::to_string(p.num_heads) +
                                     ") must be a positive multiple of num_kv_heads (" +
                                     std::to_string(p.num_kv_heads) + ")");
  if (p.sparse_mode != 0 && p.sparse_mode != 2 && p.sparse_mode != 3 && p.sparse_mode != 4)
    return fail(SWA_ERR_INVALID, "The sparse_mode value should be 0, 2, 3 or 4, but got " +
                                     std::to_string(p.sparse_mode));
  if (!std::isfinite(p.scale)) return fail(SWA_ERR_INVALID, "scale must be finite");
  // the sum of two int64 values, taken without overflow
  if (p.sparse_mode == 4 && static_cast<__int128>(p.pre_tokens) + p.next_tokens < 0)
    return fail(SWA_ERR_INVALID, "pre_tokens + next_tokens must be >= 0 in sparse_mode 4 "
                                 "(otherwise every row is empty)");
  return parse_seqs(p, seqs, end_q, end_kv);
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t max_items_fwd(int64_t num_seqs, int64_t t_q) {
  return ceil_div(t_q, FWD_BM) + num_seqs;
}
int64_t max_items_bwd(int64_t num_seqs, int64_t t_kv) {
  return ceil_div(t_kv, BWD_BN) + num_seqs;
}
int64_t max_items_dq(int64_t num_seqs, int64_t t_q) {
  return ceil_div(t_q, DQ_BM) + num_seqs;
}

// Forward workspace: the schedule (items, a work-list code per (item, head)
// unit, the work-list offsets).
size_t fwd_workspace(int64_t num_seqs, int64_t t_q, int64_t n) {
  const int64_t n_it = max_items_fwd(num_seqs, t_q);
  return align256(sizeof(Item) * n_it + sizeof(int32_t) * (n_it * n + kMaxGrid + 1));
}

// Backward workspace: schedule (dK/dV items, then dQ items, work lists) | D | lse2.
struct BwdLayout {
  size_t items, drow, lse2, total;
};

BwdLayout bwd_layout(int64_t num_seqs, int64_t t_q, int64_t t_kv, int64_t n) {
  BwdLayout l;
  l.items = 0;
  // schedule: the items of both kernels, their work lists (a code per
  // (item, head) unit) and the work-list offsets
  const int64_t n_it = max_items_bwd(num_seqs, t_kv) + max_items_dq(num_seqs, t_q);
  l.drow = align256(sizeof(Item) * n_it + sizeof(int32_t) * (n_it * n + 2 * (kMaxGrid + 1)));
  l.lse2 = l.drow + align256(sizeof(float) * t_q * n);
  l.total = l.lse2 + align256(sizeof(float) * t_q * n);
  return l;
}

Band seq_band(const Problem& p, const Seq& s) {
  switch (p.sparse_mode) {
    case 2: return Band{true, kWide, 0};                 // j <= i
    case 3: return Band{true, kWide, s.skv - s.sq};      // j - i <= Skv - Sq
    // a band reach beyond kWide covers every key of any sequence (T <= 2^20);
    // clamping it keeps the schedules' index arithmetic free of overflow
    case 4: return Band{true, std::max(-kWide, std::min(kWide, p.pre_tokens)),
                        std::max(-kWide, std::min(kWide, p.next_tokens))};
    default: return Band{false, kWide, kWide};
  }
}

int32_t clamp_window(int64_t x) {
  const int64_t lim = int64_t(1) << 30;
  return static_cast<int32_t>(std::max(-lim, std::min(lim, x)));
}

// Item fields shared by every schedule
Item make_item(const Problem& p, const Seq& s, int64_t block) {
  const Band bd = seq_band(p, s);
  Item it{};
  it.q_base = static_cast<int32_t>(s.q0);
  it.kv_base = static_cast<int32_t>(s.k0);
  it.sq = static_cast<int32_t>(s.sq);
  it.skv = static_cast<int32_t>(s.skv);
  it.block = static_cast<int32_t>(block);
  it.seq = s.b;
  it.band[0] = clamp_window(bd.pre);
  it.band[1] = clamp_window(bd.next);
  it.drop_base = s.drop_base;
  it.tiles[1] = pack_range(1, 0);
  it.full[1] = pack_range(1, 0);
  return it;
}

// Forward schedule: one item per block of FWD_BM query rows, made of two
// halves of FWD_HALF rows with their own key-tile ranges (tiles of FWD_BN).
// For a block of rows, a tile is visited iff some (i < Sq, j < Skv) in it is
// allowed, and is "full" iff the whole block x FWD_BN tile lies inside the
// sequence and inside the band.
void forward_range(const Problem& p, const Seq& s, int64_t r0, int64_t* lo, int64_t* hi,
                   int64_t* flo, int64_t* fhi) {
  const int64_t BM = FWD_HALF, BN = FWD_BN;
  *lo = 1, *hi = 0, *flo = 1, *fhi = 0;
  if (r0 >= s.sq || s.skv == 0) return;
  const int64_t r1 = std::min(r0 + BM, s.sq) - 1;
  const Band bd = seq_band(p, s);
  int64_t jlo = 0, jhi = s.skv - 1;
  if (bd.on) {
    jlo = std::max<int64_t>(0, r0 - bd.pre);
    jhi = std::min<int64_t>(s.skv - 1, r1 + bd.next);
  }
  if (jlo > jhi) return;
  *lo = jlo / BN;
  *hi = jhi / BN;
  if (r0 + BM <= s.sq) {
    *flo = *lo;
    *fhi = std::min(*hi, s.skv / BN - 1);
    if (bd.on) {
      *flo = std::max(*flo, ceil_div(r0 + BM - 1 - bd.pre, BN));
      *fhi = std::min(*fhi, floor_div(r0 + bd.next - BN + 1, BN));
    }
  }
}

void schedule_forward(const Problem& p, const std::vector<Seq>& seqs, std::vector<Item>& items) {
  items.clear();
  for (const Seq& s : seqs) {
    if (s.sq == 0) continue;
    const int64_t nqb = ceil_div(s.sq, FWD_BM);
    for (int64_t qb = 0; qb < nqb; ++qb) {
      Item it = make_item(p, s, qb);
      for (int half = 0; half < 2; ++half) {
        int64_t lo, hi, flo, fhi;
        forward_range(p, s, qb * FWD_BM + half * FWD_HALF, &lo, &hi, &flo, &fhi);
        it.tiles[half] = pack_range(lo, hi);
        it.full[half] = pack_range(flo, fhi);
      }
      items.push_back(it);
    }
  }
}

// Backward dK/dV schedule: one item per block of BWD_BN keys; query tiles of
// BWD_BM rows.
void schedule_backward(const Problem& p, const std::vector<Seq>& seqs,
                       std::vector<Item>& items) {
  items.clear();
  const int64_t BN = BWD_BN, BM = BWD_BM;
  for (const Seq& s : seqs) {
    if (s.skv == 0) continue;
    const Band bd = seq_band(p, s);
    const int64_t nkb = ceil_div(s.skv, BN);
    for (int64_t kb = 0; kb < nkb; ++kb) {
      const int64_t k0 = kb * BN, k1 = std::min(k0 + BN, s.skv) - 1;
      int64_t lo = 1, hi = 0, flo = 1, fhi = 0;
      if (s.sq > 0) {
        int64_t ilo = 0, ihi = s.sq - 1;
        if (bd.on) {
          ilo = std::max<int64_t>(0, k0 - bd.next);
          ihi = std::min<int64_t>(s.sq - 1, k1 + bd.pre);
        }
        if (ilo <= ihi) {
          lo = ilo / BM;
          hi = ihi / BM;
          if (k0 + BN <= s.skv) {
            flo = lo;
            fhi = std::min(hi, s.sq / BM - 1);
            if (bd.on) {
              flo = std::max(flo, ceil_div(k0 + BN - 1 - bd.next, BM));
              fhi = std::min(fhi, floor_div(k0 + bd.pre - BM + 1, BM));
            }
          }
        }
      }
      Item it = make_item(p, s, kb);
      it.tiles[0] = pack_range(lo, hi);
      it.full[0] = pack_range(flo, fhi);
      items.push_back(it);
    }
  }
}

// dQ schedule: one item per block of DQ_BM query rows, with
// the key-tile range of forward_range (tiles of FWD_BN).
void schedule_dq(const Problem& p, const std::vector<Seq>& seqs, std::vector<Item>& items) {
  items.clear();
  for (const Seq& s : seqs) {
    if (s.sq == 0) continue;
    const int64_t nqb = ceil_div(s.sq, DQ_BM);
    for (int64_t qb = 0; qb < nqb; ++qb) {
      int64_t lo, hi, flo, fhi;
      forward_range(p, s, qb * DQ_BM, &lo, &hi, &flo, &fhi);
      Item it = make_item(p, s, qb);
      it.tiles[0] = pack_range(lo, hi);
      it.full[0] = pack_range(flo, fhi);
      items.push_back(it);
    }
  }
}

int range_lo(int32_t r) { return r & 0xffff; }
int range_hi(int32_t r) { return (r >> 16) & 0xffff; }
int64_t range_len(int32_t r) {
  const int lo = range_lo(r), hi = range_hi(r);
  return hi >= lo ? hi - lo + 1 : 0;
}
// Work of an item: its longer range (the two halves of a forward item run
// side by side).
int64_t cost(const Item& it) { return std::max(range_len(it.tiles[0]), range_len(it.tiles[1])); }

// Longest item first (stable, so equal-cost blocks of one sequence stay in
// order and neighbouring query blocks, which read the same key/value tiles,
// run close together).
void order_items(std::vector<Item>& items) {
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& a, const Item& b) { return cost(a) > cost(b); });
}

// Static work lists of the persistent kernels: one workgroup per compute
// unit, each running a list of (item, head) units.  The units, head-major
// (heads, then the items longest first, so neighbouring blocks of a head are
// neighbours), are cut into 8 contiguous ranges of equal cost, one per XCD
// (workgroups are dispatched round-robin over the 8 XCDs, so workgroup w
// runs on XCD w % 8 and keeps the key/value tiles its range shares in that
// XCD's L2).  Within a range the units are taken longest first and each goes
// to the XCD's least loaded workgroup (longest-processing-time-first).
struct WorkList {
  std::vector<int32_t> code;  // units grouped by workgroup
  std::vector<int32_t> off;   // grid + 1 offsets into code
  int grid = 0;
};

// Cost of a unit in tile units (x10): masked tiles take about 1.4 times a
// mask-free one, and each unit adds a switch of about 1.5 tiles.
int64_t unit_cost(const Item& it, int halves) {
  int64_t c = 15;
  for (int h = 0; h < halves; ++h) {
    const int64_t n = range_len(it.tiles[h]), f = range_len(it.full[h]);
    c = std::max(c, 15 + 10 * n + 4 * (n - f));
  }
  return c;
}

void build_worklist(const std::vector<Item>& items, int64_t heads, int n_cu, int halves,
                    WorkList& wl) {
  const int64_t n_units = static_cast<int64_t>(items.size()) * heads;
  wl.grid = static_cast<int>(std::min<int64_t>(std::min(n_cu, kMaxGrid), n_units));
  wl.code.clear();
  wl.off.assign(wl.grid + 1, 0);
  if (wl.grid == 0) return;
  std::vector<int64_t> cost(items.size());
  for (size_t i = 0; i < items.size(); ++i) cost[i] = unit_cost(items[i], halves);
  // XCD ranges (all workgroups form one range unless the grid is a multiple of 8)
  const int nx = wl.grid % 8 == 0 ? 8 : 1;
  int64_t total = 0;
  for (int64_t c : cost) total += c * heads;
  std::vector<std::vector<int32_t>> per_wg(wl.grid);
  int64_t u = 0, acc = 0;
  for (int x = 0; x < nx; ++x) {
    // units [u, end) of the head-major order: cumulative cost up to (x + 1) / nx of the total
    const int64_t target = total * (x + 1) / nx;
    std::vector<std::pair<int64_t, int32_t>> range;  // (cost, code)
    while (u < n_units && (acc < target || x == nx - 1)) {
      const int64_t head = u / static_cast<int64_t>(items.size());
      const int64_t item = u - head * static_cast<int64_t>(items.size());
      range.emplace_back(cost[item], work_code(item, head));
      acc += cost[item];
      ++u;
    }
    std::stable_sort(range.begin(), range.end(),
                     [](const std::pair<int64_t, int32_t>& a, const std::pair<int64_t, int32_t>& b) {
                       return a.first > b.first;
                     });
    // least loaded workgroup of this XCD (ties: lowest index)
    std::vector<std::pair<int64_t, int>> load;  // (load, wg)
    for (int w = x; w < wl.grid; w += nx) load.emplace_back(0, w);
    auto cmp = [](const std::pair<int64_t, int>& a, const std::pair<int64_t, int>& b) {
      return a.first != b.first ? a.first > b.first : a.second > b.second;
    };
    std::make_heap(load.begin(), load.end(), cmp);
    for (const auto& r : range) {
      std::pop_heap(load.begin(), load.end(), cmp);
      load.back().first += r.first;
      per_wg[load.back().second].push_back(r.second);
      std::push_heap(load.begin(), load.end(), cmp);
    }
  }
  // Each workgroup runs its units shortest first: the workgroups of an XCD
  // then reach their unit switches (where the next unit's rows are loaded) at
  // different times instead of all together after equal-length units.
  for (int w = 0; w < wl.grid; ++w) {
    std::stable_sort(per_wg[w].begin(), per_wg[w].end(), [&](int32_t a, int32_t b) {
      return cost[a & 0xffff] < cost[b & 0xffff];
    });
    wl.off[w] = static_cast<int32_t>(wl.code.size());
    wl.code.insert(wl.code.end(), per_wg[w].begin(), per_wg[w].end());
  }
  wl.off[wl.grid] = static_cast<int32_t>(wl.code.size());
}

// Pinned staging buffers for uploading the schedule.  A slot is reused only
// after the copy recorded behind it has completed.
struct Staging {
  std::mutex mu;
  struct Slot {
    void* host = nullptr;
    size_t cap = 0;
    void* event = nullptr;
    bool pending = false;
  } slots[8];
  unsigned next = 0;
};
Staging g_staging;

swa_status upload(const void* data, size_t bytes, void* dst, void* stream) {
  if (bytes == 0) return SWA_OK;
  std::lock_guard<std::mutex> lock(g_staging.mu);
  Staging::Slot& s = g_staging.slots[g_staging.next++ % 8];
  int e = 0;
  if (s.pending) {
    if ((e = hip_event_sync(s.event)) != 0) return fail(SWA_ERR_HIP, hip_error_string(e));
    s.pending = false;
  }
  if (s.cap < bytes) {
    if (s.host) hip_pinned_free(s.host);
    s.host = nullptr;
    s.cap = 0;
    const size_t cap = std::max<size_t>(bytes, 64 * 1024);
    if ((e = hip_pinned_alloc(&s.host, cap)) != 0) return fail(SWA_ERR_HIP, hip_error_string(e));
    s.cap = cap;
  }
  if (!s.event && (e = hip_event_create(&s.event)) != 0)
    return fail(SWA_ERR_HIP, hip_error_string(e));
  std::memcpy(s.host, data, bytes);
  if ((e = hip_memcpy_h2d_async(dst, s.host, bytes, stream)) != 0)
    return fail(SWA_ERR_HIP, hip_error_string(e));
  if ((e = hip_event_record(s.event, stream)) != 0) return fail(SWA_ERR_HIP, hip_error_string(e));
  s.pending = true;
  return SWA_OK;
}

// Upload for the entry point that allocates nothing: the table goes straight
// from host memory into the device's scratch (a copy from pageable memory,
// which the HIP runtime completes before returning, so no staging buffer is
// kept); it is skipped when the last table written to that device's scratch
// is the same, since only this entry point writes the table there.
struct NoAllocTables {
  std::mutex mu;
  std::vector<uint8_t> last[64];
};
NoAllocTables g_noalloc;

swa_status upload_noalloc(const std::vector<uint8_t>& blob, void* dst, int device, void* stream) {
  if (blob.empty()) return SWA_OK;
  std::lock_guard<std::mutex> lock(g_noalloc.mu);
  std::vector<uint8_t>& last = g_noalloc.last[device];
  if (last == blob) return SWA_OK;
  last.clear();  // unknown contents until the copy has succeeded
  const int e = hip_memcpy_h2d_async(dst, blob.data(), blob.size(), stream);
  if (e != 0) return fail(SWA_ERR_HIP, hip_error_string(e));
  last = blob;
  return SWA_OK;
}

// Append the bytes of v to a schedule blob; returns the offset where they start.
template <typename T>
size_t append(std::vector<uint8_t>& blob, const std::vector<T>& v) {
  const size_t at = blob.size();
  blob.resize(at + sizeof(T) * v.size());
  if (!v.empty()) std::memcpy(blob.data() + at, v.data(), sizeof(T) * v.size());
  return at;
}

// ---- schedules as laid out in device memory
//
// A call's schedule is one contiguous blob: per kernel, its items, then
// (persistent kernels) its work-list codes and offsets.
struct SchedLayout {
  size_t bytes = 0;
  size_t at_items[2] = {0, 0};
  int32_t n_items[2] = {0, 0};
  size_t at_code[2] = {0, 0}, at_off[2] = {0, 0};
  int32_t grid[2] = {0, 0};
};

void build_forward_schedule(const Problem& p, const std::vector<Seq>& seqs, int n_cu,
                            std::vector<uint8_t>& blob, SchedLayout& L) {
  std::vector<Item> items;
  schedule_forward(p, seqs, items);
  order_items(items);
  WorkList wl;
  build_worklist(items, p.num_heads, n_cu, 2, wl);
  blob.clear();
  L = SchedLayout{};
  L.at_items[0] = append(blob, items);
  L.at_code[0] = append(blob, wl.code);
  L.at_off[0] = append(blob, wl.off);
  L.n_items[0] = static_cast<int32_t>(items.size());
  L.grid[0] = wl.grid;
  L.bytes = blob.size();
}

// Backward: kernel 0 = dK/dV, kernel 1 = dQ; work lists for the persistent
// bf16 kernels (the fp32 kernels run one workgroup per unit).
void build_backward_schedule(const Problem& p, const std::vector<Seq>& seqs, int n_cu,
                             std::vector<uint8_t>& blob, SchedLayout& L) {
  std::vector<Item> items, dq_items;
  schedule_backward(p, seqs, items);
  order_items(items);
  schedule_dq(p, seqs, dq_items);
  order_items(dq_items);
  WorkList wl_kv, wl_dq;
  if (p.dtype == SWA_DTYPE_BF16) {
    build_worklist(items, p.num_kv_heads, n_cu, 1, wl_kv);
    build_worklist(dq_items, p.num_heads, n_cu, 1, wl_dq);
  }
  blob.clear();
  L = SchedLayout{};
  L.at_items[0] = append(blob, items);
  L.at_items[1] = append(blob, dq_items);
  L.at_code[0] = append(blob, wl_kv.code);
  L.at_code[1] = append(blob, wl_dq.code);
  L.at_off[0] = append(blob, wl_kv.off);
  L.at_off[1] = append(blob, wl_dq.off);
  L.n_items[0] = static_cast<int32_t>(items.size());
  L.n_items[1] = static_cast<int32_t>(dq_items.size());
  L.grid[0] = wl_kv.grid;
  L.grid[1] = wl_dq.grid;
  L.bytes = blob.size();
}

// Library-owned device copies of recent schedules, keyed by everything a
// schedule depends on, so that repeated calls on the same problem neither
// rebuild nor upload it.  An entry is written once, by a synchronous copy,
// before any kernel reads it, and is freed only after its device is idle.
// A call pins the entry it uses from the lookup until its kernels are
// enqueued: another thread frees only unpinned entries (the wait for the
// device to be idle then covers every kernel already enqueued on it), and an
// entry dropped while pinned (cache disabled) is freed by its last unpin.
struct ScheduleCache {
  struct Entry {
    std::vector<int64_t> key;
    int device;
    void* dev;
    size_t bytes;
    SchedLayout layout;
    uint64_t used;
    uint64_t id;
    int pins;
    bool dropped;  // no longer found by lookups; freed at the last unpin
  };
  std::mutex mu;
  std::vector<Entry> entries;
  uint64_t tick = 0;
  uint64_t next_id = 0;
  size_t total = 0;
  bool enabled = true;
};
ScheduleCache g_cache;

// Frees entry i (its device idle first) and removes it; the lock is held.
int cache_free_entry(size_t i) {
  ScheduleCache::Entry& en = g_cache.entries[i];
  const int e = hip_device_free(en.device, en.dev);
  if (e != 0) return e;
  g_cache.total -= en.bytes;
  g_cache.entries.erase(g_cache.entries.begin() + i);
  return 0;
}

// The pin of one call on a cache entry (id 0: none), released when the call
// returns, after its kernels have been enqueued.
struct SchedulePin {
  uint64_t id = 0;
  SchedulePin() = default;
  SchedulePin(const SchedulePin&) = delete;
  SchedulePin& operator=(const SchedulePin&) = delete;
  ~SchedulePin() {
    if (!id) return;
    std::lock_guard<std::mutex> lock(g_cache.mu);
    for (size_t i = 0; i < g_cache.entries.size(); ++i) {
      ScheduleCache::Entry& en = g_cache.entries[i];
      if (en.id != id) continue;
      if (--en.pins == 0 && en.dropped) cache_free_entry(i);  // (a failure leaves it listed)
      return;
    }
  }
};
constexpr size_t kCacheEntries = 64;
constexpr size_t kCacheBytes = size_t(256) << 20;

std::vector<int64_t> schedule_key(int kind, int device, int n_cu, const Problem& p) {
  std::vector<int64_t> k = {kind, device, n_cu, p.dtype, p.head_dim, p.num_heads,
                            p.num_kv_heads, p.sparse_mode, p.pre_tokens, p.next_tokens,
                            p.t_q, p.t_kv, p.num_seqs};
  k.insert(k.end(), p.cu_q, p.cu_q + p.num_seqs);
  k.insert(k.end(), p.cu_kv, p.cu_kv + p.num_seqs);
  return k;
}

// Device schedule of this call: the cached copy, a new cached copy, or
// (cache disabled or full of live entries that cannot be freed, allocation
// failure, or the entry point that allocates nothing) the blob uploaded into
// `ws` (noalloc_device >= 0: that device's fixed scratch).
swa_status place_schedule(int kind, const Problem& p, const std::vector<Seq>& seqs, char* ws,
                          int noalloc_device, void* stream, const char** dev, SchedLayout* L,
                          SchedulePin* pin) {
  int n_cu = 0, device = 0, e = 0;
  if ((e = hip_cu_count(stream, &n_cu)) != 0) return fail(SWA_ERR_HIP, hip_error_string(e));
  if ((e = hip_stream_device(stream, &device)) != 0) return fail(SWA_ERR_HIP, hip_error_string(e));
  auto build = [&](std::vector<uint8_t>& blob) {
    if (kind == 0)
      build_forward_schedule(p, seqs, n_cu, blob, *L);
    else
      build_backward_schedule(p, seqs, n_cu, blob, *L);
  };
  std::vector<uint8_t> blob;
  if (noalloc_device >= 0) {
    build(blob);
    *dev = ws;
    return upload_noalloc(blob, ws, noalloc_device, stream);
  }
  std::vector<int64_t> key;
  {
    std::lock_guard<std::mutex> lock(g_cache.mu);
    if (g_cache.enabled) {
      key = schedule_key(kind, device, n_cu, p);
      for (ScheduleCache::Entry& en : g_cache.entries) {
        if (!en.dropped && en.device == device && en.key == key) {
          en.used = ++g_cache.tick;
          ++en.pins;
          pin->id = en.id;
          *dev = static_cast<const char*>(en.dev);
          *L = en.layout;
          return SWA_OK;
        }
      }
    }
  }
  build(blob);
  if (!key.empty() && !blob.empty() && blob.size() <= kCacheBytes / 4) {
    std::lock_guard<std::mutex> lock(g_cache.mu);
    // make room: least recently used unpinned entry first
    while (g_cache.enabled && (g_cache.entries.size() >= kCacheEntries ||
                               g_cache.total + blob.size() > kCacheBytes)) {
      size_t lru = g_cache.entries.size();
      for (size_t i = 0; i < g_cache.entries.size(); ++i)
        if (g_cache.entries[i].pins == 0 &&
            (lru == g_cache.entries.size() || g_cache.entries[i].used < g_cache.entries[lru].used))
          lru = i;
      if (lru == g_cache.entries.size() || cache_free_entry(lru) != 0) break;
    }
    void* d = nullptr;
    if (g_cache.enabled && g_cache.entries.size() < kCacheEntries &&
        g_cache.total + blob.size() <= kCacheBytes && hip_device_alloc(device, &d, blob.size()) == 0) {
      if (hip_memcpy_h2d_sync(device, d, blob.data(), blob.size()) == 0) {
        const uint64_t id = ++g_cache.next_id;
        g_cache.entries.push_back(ScheduleCache::Entry{std::move(key), device, d, blob.size(), *L,
                                                       ++g_cache.tick, id, 1, false});
        g_cache.total += blob.size();
        pin->id = id;
        *dev = static_cast<const char*>(d);
        return SWA_OK;
      }
      hip_device_free(device, d);
    }
  }
  *dev = ws;
  return upload(blob.data(), blob.size(), ws, stream);
}

Problem make_problem(const int64_t* cu_q, const int64_t* cu_kv, int64_t num_seqs, int64_t t_q,
                     int64_t t_kv, int64_t n, int64_t nkv, int64_t d, int32_t dtype,
                     double scale, int64_t pre, int64_t next, int64_t mode) {
  Problem p;
  p.num_seqs = num_seqs;
  p.t_q = t_q;
  p.t_kv = t_kv;
  p.num_heads = n;
  p.num_kv_heads = nkv;
  p.head_dim = d;
  p.dtype = dtype;
  p.scale = scale;
  p.pre_tokens = pre;
  p.next_tokens = next;
  p.sparse_mode = mode;
  p.cu_q = cu_q;
  p.cu_kv = cu_kv;
  p.drop_mask = nullptr;
  p.drop_mask_bytes = 0;
  p.keep_prob = 1.0;
  return p;
}

size_t elem_bytes(int32_t dtype) { return dtype == SWA_DTYPE_FP32 ? 4 : 2; }

// Optional per-kernel timing with HIP events (swa_profile_enable/read).
enum KernelKind { K_FWD = 0, K_BWD_PRE = 1, K_BWD = 2, K_FILL = 4, K_BWD_DQ = 5, K_KINDS = 6 };
struct Profiler {
  std::mutex mu;
  bool on = false;
  struct Rec {
    int kind;
    void* start;
    void* stop;
  };
  std::vector<Rec> recs;
  std::vector<void*> pool;
};
Profiler g_prof;

void* prof_event() {
  void* ev = nullptr;
  if (!g_prof.pool.empty()) {
    ev = g_prof.pool.back();
    g_prof.pool.pop_back();
  } else if (hip_event_create_timed(&ev) != 0) {
    ev = nullptr;
  }
  return ev;
}

// Launch `fn` and, if timing is on, bracket it with events on `stream`.
template <typename F>
int timed_launch(int kind, void* stream, F&& fn) {
  bool on;
  {
    std::lock_guard<std::mutex> lock(g_prof.mu);
    on = g_prof.on;
  }
  if (!on) return fn();
  void *a = nullptr, *b = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_prof.mu);
    a = prof_event();
    b = prof_event();
  }
  if (a) hip_event_record(a, stream);
  const int e = fn();
  if (b) hip_event_record(b, stream);
  std::lock_guard<std::mutex> lock(g_prof.mu);
  if (a && b) g_prof.recs.push_back(Profiler::Rec{kind, a, b});
  return e;
}

// Kernel operands of the dropout mask (words null: no dropout).
DropArgs drop_args(const Problem& p) {
  DropArgs d{static_cast<const uint32_t*>(p.drop_mask),
             static_cast<int64_t>(p.drop_mask_bytes / 4), static_cast<float>(1.0 / p.keep_prob),
             static_cast<float>(std::log2(p.keep_prob))};
  return d;
}

}  // namespace
}  // namespace swa

using namespace swa;

extern "C" {

const char* swa_last_error(void) { return g_err.c_str(); }

swa_status swa_forward_workspace_size(int64_t num_seqs, int64_t t_q, int64_t t_kv,
                                      int64_t num_heads, int64_t head_dim, int32_t dtype,
                                      size_t* bytes) {
  if (!bytes) return fail(SWA_ERR_NULLPTR, "bytes is NULL");
  swa_status s = check_sizes(num_seqs, t_q, t_kv, num_heads, head_dim, dtype);
  if (s != SWA_OK) return s;
  *bytes = fwd_workspace(num_seqs, t_q, num_heads);
  return SWA_OK;
}

swa_status swa_backward_workspace_size(int64_t num_seqs, int64_t t_q, int64_t t_kv,
                                       int64_t num_heads, int64_t head_dim, int32_t dtype,
                                       size_t* bytes) {
  if (!bytes) return fail(SWA_ERR_NULLPTR, "bytes is NULL");
  swa_status s = check_sizes(num_seqs, t_q, t_kv, num_heads, head_dim, dtype);
  if (s != SWA_OK) return s;
  *bytes = bwd_layout(num_seqs, t_q, t_kv, num_heads).total;
  return SWA_OK;
}

swa_status swa_forward_ex(const void* q, const void* k, const void* v,
                          const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                          int64_t num_seqs, int64_t t_q, int64_t t_kv, int64_t num_heads,
                          int64_t num_kv_heads, int64_t head_dim, int32_t dtype, double scale,
                          int64_t pre_tokens, int64_t next_tokens, int64_t sparse_mode,
                          const void* drop_mask, size_t drop_mask_bytes, double keep_prob,
                          void* out, float* softmax_max, float* softmax_sum, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !out || !softmax_max || !softmax_sum || !workspace)
    return fail(SWA_ERR_NULLPTR, "a required tensor or the workspace is NULL");
  Problem p = make_problem(cu_seqlens_q, cu_seqlens_kv, num_seqs, t_q, t_kv, num_heads,
                           num_kv_heads, head_dim, dtype, scale, pre_tokens, next_tokens,
                           sparse_mode);
  p.drop_mask = drop_mask;
  p.drop_mask_bytes = drop_mask_bytes;
  p.keep_prob = keep_prob;
  std::vector<Seq> seqs;
  int64_t end_q = 0, end_kv = 0;
  swa_status s = validate(p, seqs, &end_q, &end_kv);
  if (s != SWA_OK) return s;
  const size_t need = fwd_workspace(num_seqs, t_q, num_heads);
  if (workspace_bytes < need)
    return fail(SWA_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                       " bytes, needs " + std::to_string(need));
  const char* sched = nullptr;
  SchedLayout SL;
  SchedulePin pin;  // released on return, after the launches
  if ((s = place_schedule(0, p, seqs, static_cast<char*>(workspace), -1, stream, &sched, &SL,
                          &pin)) != SWA_OK)
    return s;
  int e = 0;
  if (end_q < t_q) {
    FillArgs f{out, static_cast<int64_t>(elem_bytes(dtype)), num_heads * head_dim, end_q, t_q,
               softmax_max, softmax_sum, num_heads * 8};
    if ((e = timed_launch(K_FILL, stream, [&] { return launch_fill(f, stream); })) != 0)
      return fail(SWA_ERR_HIP, hip_error_string(e));
  }
  if (SL.n_items[0] > 0) {
    FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.smax = softmax_max;
    a.ssum = softmax_sum;
    a.items = reinterpret_cast<const Item*>(sched + SL.at_items[0]);
    a.n_items = SL.n_items[0];
    a.work = reinterpret_cast<const int32_t*>(sched + SL.at_code[0]);
    a.work_off = reinterpret_cast<const int32_t*>(sched + SL.at_off[0]);
    a.n_wg = SL.grid[0];
    a.num_heads = static_cast<int32_t>(num_heads);
    a.num_kv_heads = static_cast<int32_t>(num_kv_heads);
    a.scale_log2 = static_cast<float>(scale * 1.4426950408889634);
    a.mode = static_cast<int32_t>(sparse_mode);
    a.drop = drop_args(p);
    if ((e = timed_launch(K_FWD, stream, [&] {
           return launch_forward(a, dtype, static_cast<int>(head_dim), stream);
         })) != 0)
      return fail(SWA_ERR_HIP, hip_error_string(e));
  }
  return SWA_OK;
}

swa_status swa_forward(const void* q, const void* k, const void* v, const int64_t* cu_seqlens_q,
                       const int64_t* cu_seqlens_kv, int64_t num_seqs, int64_t t_q,
                       int64_t t_kv, int64_t num_heads, int64_t head_dim, int32_t dtype,
                       double scale, int64_t pre_tokens, int64_t next_tokens,
                       int64_t sparse_mode, void* out, float* softmax_max, float* softmax_sum,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return swa_forward_ex(q, k, v, cu_seqlens_q, cu_seqlens_kv, num_seqs, t_q, t_kv, num_heads,
                        num_heads, head_dim, dtype, scale, pre_tokens, next_tokens, sparse_mode,
                        nullptr, 0, 1.0, out, softmax_max, softmax_sum, workspace,
                        workspace_bytes, stream);
}

}  // extern "C"

namespace swa {
namespace {

// Backward device arguments (the caller's buffers).
struct BwdBuffers {
  const void *q, *k, *v, *dy, *out;
  const float *smax, *ssum;
  void *dq, *dk, *dv;
};

// The backward after validation, over a workspace laid out by L.
// noalloc_device >= 0: the workspace is that device's fixed scratch, and the
// schedule is uploaded without staging (upload_noalloc).
swa_status run_backward(const Problem& p, const std::vector<Seq>& seqs, int64_t end_q,
                        int64_t end_kv, const BwdBuffers& B, char* ws, const BwdLayout& L,
                        int noalloc_device, void* stream) {
  const int64_t t_q = p.t_q, t_kv = p.t_kv, num_heads = p.num_heads;
  const int64_t num_kv_heads = p.num_kv_heads, head_dim = p.head_dim;
  const int32_t dtype = p.dtype;
  const double scale = p.scale;
  const void *q = B.q, *k = B.k, *v = B.v, *dy = B.dy, *out = B.out;
  const float *softmax_max = B.smax, *softmax_sum = B.ssum;
  void *dq = B.dq, *dk = B.dk, *dv = B.dv;
  const int64_t sparse_mode = p.sparse_mode;
  swa_status s = SWA_OK;
  // bf16: dQ kernel (it also forms D, lse2), then dK/dV kernel;
  // fp32: preprocess (D, lse2), dK/dV kernel, dQ kernel.  No atomics.
  const bool bf16 = dtype == SWA_DTYPE_BF16;
  const char* sched = nullptr;
  SchedLayout SL;
  SchedulePin pin;  // released on return, after the launches
  if ((s = place_schedule(1, p, seqs, ws + L.items, noalloc_device, stream, &sched, &SL, &pin)) !=
      SWA_OK)
    return s;
  const size_t n_kv_items = static_cast<size_t>(SL.n_items[0]);
  int e = 0;
  float* drow = reinterpret_cast<float*>(ws + L.drow);
  float* lse2 = reinterpret_cast<float*>(ws + L.lse2);
  if (!bf16) {
    BwdPreArgs pa{dy, out, softmax_max, softmax_sum, drow, lse2, t_q * num_heads,
                  static_cast<int32_t>(num_heads), static_cast<int32_t>(t_q)};
    if ((e = timed_launch(K_BWD_PRE, stream, [&] {
           return launch_bwd_pre(pa, static_cast<int>(head_dim), stream);
         })) != 0)
      return fail(SWA_ERR_HIP, hip_error_string(e));
  }
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dy = dy;
  a.drow = drow;
  a.lse2 = lse2;
  a.out = out;
  a.smax = softmax_max;
  a.ssum = softmax_sum;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.items = reinterpret_cast<const Item*>(sched + SL.at_items[0]);
  a.n_items = SL.n_items[0];
  a.work = reinterpret_cast<const int32_t*>(sched + SL.at_code[0]);
  a.work_off = reinterpret_cast<const int32_t*>(sched + SL.at_off[0]);
  a.n_wg = SL.grid[0];
  a.num_heads = static_cast<int32_t>(num_heads);
  a.num_kv_heads = static_cast<int32_t>(num_kv_heads);
  a.t_q = static_cast<int32_t>(t_q);
  a.drop = drop_args(p);
  a.scale = static_cast<float>(scale);
  a.scale_log2 = static_cast<float>(scale * 1.4426950408889634);
  a.mode = static_cast<int32_t>(sparse_mode);
  // The dQ schedule has one item per block of query rows of every sequence,
  // even when the block attends no key (its dq rows are written as zero; the
  // bf16 dQ kernel also writes their D and lse2, read by its dK/dV kernel).
  BwdArgs b = a;
  b.items = reinterpret_cast<const Item*>(sched + SL.at_items[1]);
  b.n_items = SL.n_items[1];
  b.work = reinterpret_cast<const int32_t*>(sched + SL.at_code[1]);
  b.work_off = reinterpret_cast<const int32_t*>(sched + SL.at_off[1]);
  b.n_wg = SL.grid[1];
  if (bf16 && SL.n_items[1] > 0) {
    if ((e = timed_launch(K_BWD_DQ, stream, [&] {
           return launch_bwd_dq(b, static_cast<int>(head_dim), stream);
         })) != 0)
      return fail(SWA_ERR_HIP, hip_error_string(e));
  }
  if (n_kv_items > 0) {
    if ((e = timed_launch(K_BWD, stream, [&] {
           return launch_backward(a, dtype, static_cast<int>(head_dim), stream);
         })) != 0)
      return fail(SWA_ERR_HIP, hip_error_string(e));
  }
  if (!bf16 && SL.n_items[1] > 0) {
    if ((e = timed_launch(K_BWD_DQ, stream, [&] {
           return launch_bwd_dq_f32(b, static_cast<int>(head_dim), stream);
         })) != 0)
      return fail(SWA_ERR_HIP, hip_error_string(e));
  }
  if (end_q < t_q) {  // tokens after the last sequence
    FillArgs f{dq, static_cast<int64_t>(elem_bytes(dtype)), num_heads * head_dim, end_q, t_q,
               nullptr, nullptr, 0};
    if ((e = timed_launch(K_FILL, stream, [&] { return launch_fill(f, stream); })) != 0)
      return fail(SWA_ERR_HIP, hip_error_string(e));
  }
  if (end_kv < t_kv) {
    FillArgs f{dk, static_cast<int64_t>(elem_bytes(dtype)), num_kv_heads * head_dim, end_kv,
               t_kv, nullptr, nullptr, 0};
    if ((e = timed_launch(K_FILL, stream, [&] { return launch_fill(f, stream); })) != 0)
      return fail(SWA_ERR_HIP, hip_error_string(e));
    f.x = dv;
    if ((e = timed_launch(K_FILL, stream, [&] { return launch_fill(f, stream); })) != 0)
      return fail(SWA_ERR_HIP, hip_error_string(e));
  }
  return SWA_OK;
}

// Validation shared by the backward entry points.
swa_status backward_problem(const void* q, const void* k, const void* v, const void* dy,
                            const void* out, const float* softmax_max, const float* softmax_sum,
                            const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                            int64_t num_seqs, int64_t t_q, int64_t t_kv, int64_t num_heads,
                            int64_t num_kv_heads, int64_t head_dim, int32_t dtype, double scale,
                            int64_t pre_tokens, int64_t next_tokens, int64_t sparse_mode,
                            const void* drop_mask, size_t drop_mask_bytes, double keep_prob,
                            void* dq, void* dk, void* dv, Problem* p, std::vector<Seq>* seqs,
                            int64_t* end_q, int64_t* end_kv, BwdBuffers* B) {
  if (!q || !k || !v || !dy || !out || !softmax_max || !softmax_sum || !dq || !dk || !dv)
    return fail(SWA_ERR_NULLPTR, "a required tensor is NULL");
  *p = make_problem(cu_seqlens_q, cu_seqlens_kv, num_seqs, t_q, t_kv, num_heads, num_kv_heads,
                    head_dim, dtype, scale, pre_tokens, next_tokens, sparse_mode);
  p->drop_mask = drop_mask;
  p->drop_mask_bytes = drop_mask_bytes;
  p->keep_prob = keep_prob;
  *B = BwdBuffers{q, k, v, dy, out, softmax_max, softmax_sum, dq, dk, dv};
  return validate(*p, *seqs, end_q, end_kv);
}

}  // namespace
}  // namespace swa

extern "C" {

swa_status swa_backward_ex(const void* q, const void* k, const void* v, const void* dy,
                           const void* out, const float* softmax_max, const float* softmax_sum,
                           const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                           int64_t num_seqs, int64_t t_q, int64_t t_kv, int64_t num_heads,
                           int64_t num_kv_heads, int64_t head_dim, int32_t dtype, double scale,
                           int64_t pre_tokens, int64_t next_tokens, int64_t sparse_mode,
                           const void* drop_mask, size_t drop_mask_bytes, double keep_prob,
                           void* dq, void* dk, void* dv, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (!workspace) return fail(SWA_ERR_NULLPTR, "the workspace is NULL");
  Problem p;
  std::vector<Seq> seqs;
  int64_t end_q = 0, end_kv = 0;
  BwdBuffers B;
  swa_status s = backward_problem(q, k, v, dy, out, softmax_max, softmax_sum, cu_seqlens_q,
                                  cu_seqlens_kv, num_seqs, t_q, t_kv, num_heads, num_kv_heads,
                                  head_dim, dtype, scale, pre_tokens, next_tokens, sparse_mode,
                                  drop_mask, drop_mask_bytes, keep_prob, dq, dk, dv, &p, &seqs,
                                  &end_q, &end_kv, &B);
  if (s != SWA_OK) return s;
  const BwdLayout L = bwd_layout(num_seqs, t_q, t_kv, num_heads);
  if (workspace_bytes < L.total)
    return fail(SWA_ERR_WORKSPACE, "workspace has " + std::to_string(workspace_bytes) +
                                       " bytes, needs " + std::to_string(L.total));
  return run_backward(p, seqs, end_q, end_kv, B, static_cast<char*>(workspace), L, -1, stream);
}

swa_status swa_backward_noalloc(const void* q, const void* k, const void* v, const void* dy,
                                const void* out, const float* softmax_max,
                                const float* softmax_sum, const int64_t* cu_seqlens_q,
                                const int64_t* cu_seqlens_kv, int64_t num_seqs, int64_t t_q,
                                int64_t t_kv, int64_t num_heads, int64_t num_kv_heads,
                                int64_t head_dim, int32_t dtype, double scale,
                                int64_t pre_tokens, int64_t next_tokens, int64_t sparse_mode,
                                const void* drop_mask, size_t drop_mask_bytes, double keep_prob,
                                void* dq, void* dk, void* dv, void* stream) {
  Problem p;
  std::vector<Seq> seqs;
  int64_t end_q = 0, end_kv = 0;
  BwdBuffers B;
  swa_status s = backward_problem(q, k, v, dy, out, softmax_max, softmax_sum, cu_seqlens_q,
                                  cu_seqlens_kv, num_seqs, t_q, t_kv, num_heads, num_kv_heads,
                                  head_dim, dtype, scale, pre_tokens, next_tokens, sparse_mode,
                                  drop_mask, drop_mask_bytes, keep_prob, dq, dk, dv, &p, &seqs,
                                  &end_q, &end_kv, &B);
  if (s != SWA_OK) return s;
  const BwdLayout L = bwd_layout(num_seqs, t_q, t_kv, num_heads);
  if (L.total > kNoAllocScratchBytes)
    return fail(SWA_ERR_WORKSPACE,
                "this problem needs " + std::to_string(L.total) + " bytes of scratch; "
                "swa_backward_noalloc has a fixed " + std::to_string(kNoAllocScratchBytes) +
                " bytes per device (call swa_backward_ex with a workspace instead)");
  void* scratch = nullptr;
  int device = 0;
  const int e = noalloc_scratch(stream, &scratch, &device);
  if (e != 0) return fail(SWA_ERR_HIP, hip_error_string(e));
  return run_backward(p, seqs, end_q, end_kv, B, static_cast<char*>(scratch), L, device,
                      stream);
}

swa_status swa_backward(const void* q, const void* k, const void* v, const void* dy,
                        const void* out, const float* softmax_max, const float* softmax_sum,
                        const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                        int64_t num_seqs, int64_t t_q, int64_t t_kv, int64_t num_heads,
                        int64_t head_dim, int32_t dtype, double scale, int64_t pre_tokens,
                        int64_t next_tokens, int64_t sparse_mode, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return swa_backward_ex(q, k, v, dy, out, softmax_max, softmax_sum, cu_seqlens_q,
                         cu_seqlens_kv, num_seqs, t_q, t_kv, num_heads, num_heads, head_dim,
                         dtype, scale, pre_tokens, next_tokens, sparse_mode, nullptr, 0, 1.0,
                         dq, dk, dv, workspace, workspace_bytes, stream);
}

swa_status swa_debug_tile_schedule(const int64_t* cu_seqlens_q, const int64_t* cu_seqlens_kv,
                                   int64_t num_seqs, int64_t t_q, int64_t t_kv,
                                   int64_t head_dim, int32_t dtype, int64_t pre_tokens,
                                   int64_t next_tokens, int64_t sparse_mode, int32_t direction,
                                   int32_t* rows_out, int64_t capacity, int64_t* n_rows,
                                   int32_t* block_item, int32_t* block_tile) {
  if (!n_rows || !block_item || !block_tile)
    return fail(SWA_ERR_NULLPTR, "n_rows / block_item / block_tile is NULL");
  if (direction < 0 || direction > 2)
    return fail(SWA_ERR_INVALID,
                "direction must be 0 (forward), 1 (backward dK/dV) or 2 (backward dQ)");
  Problem p = make_problem(cu_seqlens_q, cu_seqlens_kv, num_seqs, t_q, t_kv, 1, 1, head_dim,
                           dtype, 1.0, pre_tokens, next_tokens, sparse_mode);
  std::vector<Seq> seqs;
  int64_t end_q = 0, end_kv = 0;
  swa_status s = validate(p, seqs, &end_q, &end_kv);
  if (s != SWA_OK) return s;
  std::vector<Item> items;
  if (direction == 0) {
    schedule_forward(p, seqs, items);
    *block_item = FWD_HALF;
    *block_tile = FWD_BN;
  } else if (direction == 1) {
    schedule_backward(p, seqs, items);
    *block_item = BWD_BN;
    *block_tile = BWD_BM;
  } else {
    schedule_dq(p, seqs, items);
    *block_item = DQ_BM;
    *block_tile = FWD_BN;
  }
  order_items(items);
  int64_t n = 0;
  auto emit = [&](int32_t a, int32_t b, int32_t c, int32_t d) {
    if (rows_out && n < capacity) {
      rows_out[4 * n + 0] = a;
      rows_out[4 * n + 1] = b;
      rows_out[4 * n + 2] = c;
      rows_out[4 * n + 3] = d;
    }
    ++n;
  };
  for (const Item& it : items) {
    const int halves = direction == 0 ? 2 : 1;
    for (int half = 0; half < halves; ++half) {
      const int32_t block = direction == 0 ? it.block * 2 + half : it.block;
      if (direction == 0 && static_cast<int64_t>(block) * FWD_HALF >= it.sq) continue;
      const int lo = range_lo(it.tiles[half]), hi = range_hi(it.tiles[half]);
      const int flo = range_lo(it.full[half]), fhi = range_hi(it.full[half]);
      if (hi < lo) {
        emit(it.seq, block, -1, 0);
        continue;
      }
      for (int t = lo; t <= hi; ++t) emit(it.seq, block, t, (t >= flo && t <= fhi) ? 2 : 1);
    }
  }
  *n_rows = n;
  return SWA_OK;
}

swa_status swa_schedule_cache_enable(int32_t enable) {
  std::lock_guard<std::mutex> lock(g_cache.mu);
  g_cache.enabled = enable != 0;
  if (!enable) {
    // entries in use by a call on another thread are dropped now and freed
    // when that call has enqueued its kernels
    for (size_t i = g_cache.entries.size(); i-- > 0;) {
      ScheduleCache::Entry& en = g_cache.entries[i];
      en.dropped = true;
      if (en.pins > 0) continue;
      const int e = cache_free_entry(i);
      if (e != 0) return fail(SWA_ERR_HIP, hip_error_string(e));
    }
  }
  return SWA_OK;
}

swa_status swa_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lock(g_prof.mu);
  g_prof.on = enable != 0;
  return SWA_OK;
}

swa_status swa_profile_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(SWA_ERR_NULLPTR, "total_ms / launches is NULL");
  if (kernel < 0 || kernel >= K_KINDS) return fail(SWA_ERR_INVALID, "unknown kernel kind");
  std::lock_guard<std::mutex> lock(g_prof.mu);
  double sum = 0.0;
  int64_t n = 0;
  std::vector<Profiler::Rec> keep;
  for (const Profiler::Rec& r : g_prof.recs) {
    if (r.kind != kernel) {
      keep.push_back(r);
      continue;
    }
    int e = hip_event_sync(r.stop);
    float ms = 0.f;
    if (e == 0) e = hip_event_elapsed_ms(&ms, r.start, r.stop);
    if (e != 0) return fail(SWA_ERR_HIP, hip_error_string(e));
    sum += ms;
    ++n;
    g_prof.pool.push_back(r.start);
    g_prof.pool.push_back(r.stop);
  }
  g_prof.recs.swap(keep);
  *total_ms = sum;
  *launches = n;
  return SWA_OK;
}

}  // extern "C"
