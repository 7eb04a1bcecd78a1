// jt_build_tree / jt_build_tree_variant: the best-first selection of the
// candidate tree from the per-depth partials of draft_row_scan.
//
// Method: JetSpec news piece (mlqm.cn/news/158889), tree-construction
// paragraph; JetSpec explainer (techwalker.com, "加速AI思考…"), section 五.
//
// tree_select (the default rule): one workgroup per sequence.  The best-first
//   pop order equals the B smallest keys (-score, parent index, rank) of the
//   complete tree, because a child never precedes its parent.  It is computed
//   level by level: level d keeps the best cap_d = min(W^d, B-d+1) children of
//   level d-1 (a depth-d node in the final tree is preceded by its d-1
//   ancestors, so no deeper position can be selected); the W candidate columns
//   of a level are each sorted, so the level is their merge (merge path), and
//   the sorted levels are merged the same way into the global pop order.  Once
//   B kept nodes score at or above some kept score, that score bounds the
//   selection from below and later levels keep only children at or above it.
//   All
//   arithmetic on scores is fp64 and identical to a sequential evaluation
//   except the per-depth log-sum-exp, whose summation order differs.
// tree_select_seq (the variants): a literal best-first search, described below.
#include "jt_device.h"
#include "jt_host.h"

#include <algorithm>
#include <climits>
#include <cmath>

namespace jt {

constexpr int kSelectThreads = 1024;

// Per-level capacity: a node at depth d with position i in its level has at
// least i + d - 1 predecessors in the pop order.
__host__ __device__ inline int level_cap(int d, int width, int budget) {
  long long w = 1;
  for (int k = 0; k < d && w <= budget; ++k) w *= width;
  const long long byb = static_cast<long long>(budget) - d + 1;
  const long long c = w < byb ? w : byb;
  return c < 0 ? 0 : static_cast<int>(c);
}

struct SelectLayout {
  int tot;         // sum of level capacities
  int capmax;      // max level capacity
  int wp;          // power of two >= W (lists merged per level)
  int np;          // power of two >= N (lists merged across levels)
  int mstride;     // list stride of the phase-3 merge buffers (>= 1)
  size_t off_S, off_lse, off_cval, off_ctok, off_loff, off_lcnt, off_rawa, off_rawb;
  size_t off_score, off_info, off_gidx, off_ms0, off_ms1, off_mi0, off_mi1, off_len, bytes;
};

inline SelectLayout select_layout(int depth_n, int width, int budget, int wmax) {
  SelectLayout L{};
  L.tot = 0;
  L.capmax = 1;
  for (int d = 1; d <= depth_n; ++d) {
    const int c = level_cap(d, width, budget);
    L.tot += c;
    L.capmax = std::max(L.capmax, c);
  }
  L.wp = 1;
  while (L.wp < width) L.wp <<= 1;
  L.np = 1;
  while (L.np < depth_n) L.np <<= 1;
  L.mstride = std::max(1, budget);
  const size_t mcount = std::max(static_cast<size_t>(L.wp) * L.capmax,
                                 static_cast<size_t>(L.np) * L.mstride);
  size_t o = 0;
  auto take = [&](size_t n, size_t align) { o = (o + align - 1) / align * align; size_t r = o; o += n; return r; };
  L.off_S = take(sizeof(double) * (depth_n + 1), 8);
  L.off_lse = take(sizeof(double) * depth_n, 8);
  L.off_rawa = take(sizeof(double) * L.capmax, 8);
  L.off_rawb = take(sizeof(double) * L.capmax, 8);
  L.off_score = take(sizeof(double) * std::max(1, L.tot), 8);
  L.off_ms0 = take(sizeof(double) * L.wp * L.capmax, 8);
  L.off_ms1 = take(sizeof(double) * L.wp * L.capmax, 8);
  L.off_cval = take(sizeof(float) * depth_n * wmax, 4);
  L.off_ctok = take(sizeof(int) * depth_n * wmax, 4);
  L.off_loff = take(sizeof(int) * (depth_n + 2), 4);
  L.off_lcnt = take(sizeof(int) * (depth_n + 2), 4);
  L.off_info = take(sizeof(uint32_t) * std::max(1, L.tot), 4);
  L.off_mi0 = take(sizeof(uint32_t) * mcount, 4);
  L.off_mi1 = take(sizeof(uint32_t) * mcount, 4);
  L.off_len = take(sizeof(int) * 2 * std::max(L.wp, L.np), 4);
  L.off_gidx = take(sizeof(uint16_t) * std::max(1, L.tot), 2);
  L.bytes = (o + 15) / 16 * 16;
  return L;
}

// Does kept node (d2, j) precede kept node (d, i), d2 != d, given that their
// scores are equal?  Compare the parents' keys, walking up both paths (their
// depths keep differing, so they never meet; the root precedes every node).
__device__ __noinline__ bool precedes_tied(const double* score, const uint32_t* info,
                                           const int* loff, int d2, int j, int d, int i) {
  while (true) {
    j = static_cast<int>(info[loff[d2] + j] & 0xFFFFu);
    i = static_cast<int>(info[loff[d] + i] & 0xFFFFu);
    --d2;
    --d;
    if (d2 == 0) return true;
    if (d == 0) return false;
    const double sy = score[loff[d2] + j];
    const double sx = score[loff[d] + i];
    if (sy != sx) return sy > sx;
  }
}

// Same-level order of two candidates (score, info = parent position | rank << 16).
__device__ __forceinline__ bool precedes_level(double sa, uint32_t ia, double sb, uint32_t ib) {
  if (sa != sb) return sa > sb;
  const uint32_t pa = ia & 0xFFFFu, pb = ib & 0xFFFFu;
  if (pa != pb) return pa < pb;
  return (ia >> 16) < (ib >> 16);
}

// Merge path: number of elements of A among the first o outputs of merge(A, B)
// under a strict order (A[i-1] precedes B[o-i] holds exactly for i <= answer).
template <typename Prec>
__device__ __forceinline__ int co_rank(int o, int la, int lb, Prec prec_ab) {
  int lo = max(0, o - lb), hi = min(o, la);
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (prec_ab(mid - 1, o - mid)) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Wave argmax of (value, id) under `better`, through DPP lane moves into lane
// 63, then broadcast: quad swaps, rotations by 4 and 8 inside each row of 16
// lanes, row broadcasts 15 and 31 (the order is total, so any combination
// order gives the same winner).  Lanes a move does not reach keep their pair.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_better(float& v, int& id) {
  const float ov = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                         CTRL, ROW_MASK, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(id, id, CTRL, ROW_MASK, 0xF, false);
  if (better(ov, oi, v, id)) { v = ov; id = oi; }
}

__device__ __forceinline__ void wave_best_all(float& v, int& id) {
  dpp_better<0xB1, 0xF>(v, id);   // quad_perm [1, 0, 3, 2]
  dpp_better<0x4E, 0xF>(v, id);   // quad_perm [2, 3, 0, 1]
  dpp_better<0x124, 0xF>(v, id);  // row_ror 4
  dpp_better<0x128, 0xF>(v, id);  // row_ror 8
  dpp_better<0x142, 0xA>(v, id);  // row_bcast 15 into rows 1 and 3
  dpp_better<0x143, 0xC>(v, id);  // row_bcast 31 into rows 2 and 3
  v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kWave - 1));
  id = __builtin_amdgcn_readlane(id, kWave - 1);
}

// Merge the chunk partials of every depth of sequence seq (one wave a depth;
// each lane holds one chunk's sorted candidates in registers): lse[d], the
// top-W (cval, ctok [d * WMAX + r]) and, when part_ent is given, the entropy
// ent[d] = log S - T / S with S = sum exp(x - max), T = sum exp(x - max)(x - max).
template <int WMAX>
__device__ void merge_depth_partials(const float* __restrict__ part_max,
                                     const double* __restrict__ part_sum,
                                     const double* __restrict__ part_ent,
                                     const float* __restrict__ part_val,
                                     const int* __restrict__ part_idx, int chunks, int depth_n,
                                     int width, int seq, double* lse, double* ent, float* cval,
                                     int* ctok, int32_t* err, int nwaves) {
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  for (int d = wv; d < depth_n; d += nwaves) {
    const size_t row = static_cast<size_t>(seq) * depth_n + d;
    const bool act = lane < chunks;
    const float mc = act ? part_max[row * chunks + lane] : -INFINITY;
    const double sc = act ? part_sum[row * chunks + lane] : 0.0;
    float hv[WMAX];
    int hid[WMAX];
#pragma unroll
    for (int k = 0; k < WMAX; ++k) {
      const bool ok = act && k < width;
      hv[k] = ok ? part_val[(row * chunks + lane) * width + k] : -INFINITY;
      hid[k] = ok ? part_idx[(row * chunks + lane) * width + k] : INT32_MAX;
    }
    float M = mc;
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, shfl_xor(M, o));
    const double scale =
        (mc == -INFINITY) ? 0.0 : exp(static_cast<double>(mc) - static_cast<double>(M));
    double contrib = sc * scale;
    for (int o = 32; o > 0; o >>= 1) contrib += shfl_xor_f64(contrib, o);
    double tsum = 0.0;
    if (part_ent) {
      // the chunk's terms were taken about its own max mc: shift them to M
      const double tc = act ? part_ent[row * chunks + lane] : 0.0;
      tsum = (mc == -INFINITY)
                 ? 0.0
                 : scale * (tc + (static_cast<double>(mc) - static_cast<double>(M)) * sc);
      for (int o = 32; o > 0; o >>= 1) tsum += shfl_xor_f64(tsum, o);
    }
    if (lane == 0) {
      if (M == -INFINITY) {
        report(err, JT_DERR_BAD_LOGIT);
        lse[d] = 0.0;
        if (ent) ent[d] = 0.0;
      } else {
        lse[d] = static_cast<double>(M) + log(contrib);
        if (ent) ent[d] = log(contrib) - tsum / contrib;
      }
    }
    for (int r = 0; r < width; ++r) {
      float bv = hv[0];
      int bi = hid[0];
      wave_best_all(bv, bi);
      if (hid[0] == bi && bi != INT32_MAX) {  // this lane's head won: pop it
#pragma unroll
        for (int k = 0; k + 1 < WMAX; ++k) { hv[k] = hv[k + 1]; hid[k] = hid[k + 1]; }
        hv[WMAX - 1] = -INFINITY;
        hid[WMAX - 1] = INT32_MAX;
      }
      if (lane == 0) { cval[d * WMAX + r] = bv; ctok[d * WMAX + r] = bi; }
    }
  }
}

// One workgroup per sequence.
//  phase 1: per depth, merge the chunk partials (lse, top-W).
//  phase 2: per level d, the W candidate columns (children of the sorted level
//    d-1 by rank k; each column sorted, pruned to the first cap_d/(k+1) rows)
//    are merged pairwise (merge path, log2 W rounds) into the sorted level,
//    truncated to cap_d.
//  phase 3: the sorted levels are merged pairwise (log2 N rounds, truncated to
//    B) under the global key; the merged position is the node index.
//  phase 4: write parent/token/depth/score in node order.
template <int WMAX>
__global__ __launch_bounds__(kSelectThreads) void tree_select(
    const float* __restrict__ part_max, const double* __restrict__ part_sum,
    const float* __restrict__ part_val, const int* __restrict__ part_idx, int chunks, int depth_n,
    int width, int budget, SelectLayout L, const int32_t* __restrict__ root_token,
    int32_t* __restrict__ parent, int32_t* __restrict__ token, int32_t* __restrict__ depth,
    double* __restrict__ score_out, int32_t* __restrict__ n_nodes, int32_t* err) {
  extern __shared__ __align__(16) unsigned char smem[];
  double* S = reinterpret_cast<double*>(smem + L.off_S);
  double* lse = reinterpret_cast<double*>(smem + L.off_lse);
  double* raw_a = reinterpret_cast<double*>(smem + L.off_rawa);
  double* raw_b = reinterpret_cast<double*>(smem + L.off_rawb);
  double* lv_score = reinterpret_cast<double*>(smem + L.off_score);
  double* ms[2] = {reinterpret_cast<double*>(smem + L.off_ms0),
                   reinterpret_cast<double*>(smem + L.off_ms1)};
  float* cval = reinterpret_cast<float*>(smem + L.off_cval);
  int* ctok = reinterpret_cast<int*>(smem + L.off_ctok);
  int* loff = reinterpret_cast<int*>(smem + L.off_loff);
  int* lcnt = reinterpret_cast<int*>(smem + L.off_lcnt);
  uint32_t* lv_info = reinterpret_cast<uint32_t*>(smem + L.off_info);
  uint32_t* mi[2] = {reinterpret_cast<uint32_t*>(smem + L.off_mi0),
                     reinterpret_cast<uint32_t*>(smem + L.off_mi1)};
  int* lens = reinterpret_cast<int*>(smem + L.off_len);  // [2][max(wp, np)]
  uint16_t* lv_gidx = reinterpret_cast<uint16_t*>(smem + L.off_gidx);
  const int lstride = max(L.wp, L.np);

  const int seq = blockIdx.x;
  const int tid = threadIdx.x;
  const int nwaves = kSelectThreads / kWave;

  // ---- phase 1: merge the chunk partials of every depth
  merge_depth_partials<WMAX>(part_max, part_sum, nullptr, part_val, part_idx, chunks, depth_n,
                             width, seq, lse, nullptr, cval, ctok, err, nwaves);
  __syncthreads();
  if (tid == 0) {
    S[0] = 0.0;
    for (int d = 0; d < depth_n; ++d) S[d + 1] = S[d] + lse[d];
    int o = 0;
    loff[0] = 0;
    lcnt[0] = 1;
    for (int d = 1; d <= depth_n; ++d) { loff[d] = o; o += level_cap(d, width, budget); }
    loff[depth_n + 1] = o;
    raw_a[0] = 0.0;
  }
  for (int x = tid; x < L.tot; x += kSelectThreads) lv_gidx[x] = 0xFFFF;
  __syncthreads();

  // ---- phase 2: level by level, the best cap_d children in key order
  double* raw_prev = raw_a;
  double* raw_cur = raw_b;
  int m_prev = 1;
  int last_level = 0;
  // A lower bound tau of the B-th best score of the tree: any score t such
  // that B kept nodes score >= t.  For the entries t of the newest level the
  // count is (position + 1) plus, per earlier level, the entries >= t (binary
  // search in its sorted list); tau is the largest entry whose count reaches
  // B.  Children scoring below tau can never be selected, and since a
  // column's scores fall with the parent position they form a suffix that is
  // cut off.  The kept lists stay prefixes of the uncut ones, so the result
  // is unchanged; deep levels usually empty out and the loop ends early.
  __shared__ int s_istar;
  double tau = -INFINITY;
  int prev_cnt = 0;
  for (int d = 1; d <= depth_n; ++d) {
    const int cap = level_cap(d, width, budget);
    if (cap <= 0 || m_prev == 0) break;
    const double Sd = S[d];
    // column k holds children (p, k) of the first len_k parents
    if (tid < L.wp) {
      int lk = tid < width ? min(m_prev, cap / (tid + 1)) : 0;
      if (tau != -INFINITY && lk > 0) {
        const double c = static_cast<double>(cval[(d - 1) * WMAX + tid]);
        int lo = 0, hi = lk;  // first parent whose child scores below tau
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((raw_prev[mid] + c) - Sd >= tau) lo = mid + 1; else hi = mid;
        }
        lk = lo;
      }
      lens[tid] = lk;
    }
    __syncthreads();
    // columns: list k at ms/mi[0] + k * cap
    for (int idx = tid; idx < L.wp * cap; idx += kSelectThreads) {
      const int k = idx / cap, p = idx % cap;
      if (p < lens[k]) {
        ms[0][idx] = (raw_prev[p] + static_cast<double>(cval[(d - 1) * WMAX + k])) - Sd;
        mi[0][idx] = static_cast<uint32_t>(p) | (static_cast<uint32_t>(k) << 16);
      }
    }
    __syncthreads();
    int src = 0;
    for (int lists = L.wp; lists > 1; lists >>= 1) {
      const int pairs = lists >> 1;
      const int* lsrc = lens + src * lstride;
      int* ldst = lens + (src ^ 1) * lstride;
      for (int idx = tid; idx < pairs * cap; idx += kSelectThreads) {
        const int q = idx / cap, o = idx % cap;
        const int la = lsrc[2 * q], lb = lsrc[2 * q + 1];
        if (o >= min(cap, la + lb)) continue;
        const double* As = ms[src] + (2 * q) * cap;
        const uint32_t* Ai = mi[src] + (2 * q) * cap;
        const double* Bs = As + cap;
        const uint32_t* Bi = Ai + cap;
        const int i = co_rank(o, la, lb, [&](int ia, int jb) {
          return precedes_level(As[ia], Ai[ia], Bs[jb], Bi[jb]);
        });
        const int j = o - i;
        const bool take_a = i < la && (j >= lb || precedes_level(As[i], Ai[i], Bs[j], Bi[j]));
        ms[src ^ 1][q * cap + o] = take_a ? As[i] : Bs[j];
        mi[src ^ 1][q * cap + o] = take_a ? Ai[i] : Bi[j];
      }
      if (tid < pairs) ldst[tid] = min(cap, lsrc[2 * tid] + lsrc[2 * tid + 1]);
      __syncthreads();
      src ^= 1;
    }
    const int m_d = lens[src * lstride];
    for (int o = tid; o < m_d; o += kSelectThreads) {
      const uint32_t inf = mi[src][o];
      lv_score[loff[d] + o] = ms[src][o];
      lv_info[loff[d] + o] = inf;
      raw_cur[o] = raw_prev[inf & 0xFFFFu] + static_cast<double>(cval[(d - 1) * WMAX + (inf >> 16)]);
    }
    if (tid == 0) {
      lcnt[d] = m_d;
      s_istar = INT_MAX;
    }
    __syncthreads();
    if (prev_cnt + m_d >= budget) {
      // count[i] = i + 1 + sum over earlier levels of their entries >= the
      // i-th entry; one (entry, earlier level) binary search per thread step,
      // summed by LDS atomics (the merge buffers are free until the next level)
      int* cnt = reinterpret_cast<int*>(mi[0]);
      for (int i = tid; i < m_d; i += kSelectThreads) cnt[i] = i + 1;
      __syncthreads();
      for (int x = tid; x < m_d * (d - 1); x += kSelectThreads) {
        const int i = x % m_d, dd = 1 + x / m_d;
        const double t = lv_score[loff[d] + i];
        const double* ls = lv_score + loff[dd];
        int lo = 0, hi = lcnt[dd];  // entries >= t form a prefix
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (ls[mid] >= t) lo = mid + 1; else hi = mid;
        }
        if (lo > 0) atomicAdd(&cnt[i], lo);
      }
      __syncthreads();
      for (int i = tid; i < m_d; i += kSelectThreads)
        if (cnt[i] >= budget) atomicMin(&s_istar, i);
      __syncthreads();
      if (s_istar != INT_MAX) tau = fmax(tau, lv_score[loff[d] + s_istar]);
    }
    prev_cnt += m_d;
    double* t = raw_prev; raw_prev = raw_cur; raw_cur = t;
    m_prev = m_d;
    last_level = d;
  }
  if (tid == 0)
    for (int d = last_level + 1; d <= depth_n; ++d) lcnt[d] = 0;
  __syncthreads();

  // ---- phase 3: merge the sorted levels into the global order
  const int B = L.mstride;
  for (int idx = tid; idx < L.np * B; idx += kSelectThreads) {
    const int l = idx / B, o = idx % B;
    if (l < depth_n && o < lcnt[l + 1])
      mi[0][idx] = (static_cast<uint32_t>(l + 1) << 16) | static_cast<uint32_t>(o);
  }
  if (tid < L.np) lens[tid] = tid < depth_n ? min(B, lcnt[tid + 1]) : 0;
  __syncthreads();
  auto prec_cross = [&](uint32_t ra, uint32_t rb) {
    const int da = static_cast<int>(ra >> 16), ia = static_cast<int>(ra & 0xFFFFu);
    const int db = static_cast<int>(rb >> 16), ib = static_cast<int>(rb & 0xFFFFu);
    const double sa = lv_score[loff[da] + ia], sb = lv_score[loff[db] + ib];
    if (sa != sb) return sa > sb;
    return precedes_tied(lv_score, lv_info, loff, da, ia, db, ib);
  };
  int src = 0;
  for (int lists = L.np; lists > 1; lists >>= 1) {
    const int pairs = lists >> 1;
    const int* lsrc = lens + src * lstride;
    int* ldst = lens + (src ^ 1) * lstride;
    for (int idx = tid; idx < pairs * B; idx += kSelectThreads) {
      const int q = idx / B, o = idx % B;
      const int la = lsrc[2 * q], lb = lsrc[2 * q + 1];
      if (o >= min(B, la + lb)) continue;
      const uint32_t* A = mi[src] + (2 * q) * B;
      const uint32_t* Bv = A + B;
      const int i = co_rank(o, la, lb, [&](int ia, int jb) { return prec_cross(A[ia], Bv[jb]); });
      const int j = o - i;
      const bool take_a = i < la && (j >= lb || prec_cross(A[i], Bv[j]));
      mi[src ^ 1][q * B + o] = take_a ? A[i] : Bv[j];
    }
    if (tid < pairs) ldst[tid] = min(B, lsrc[2 * tid] + lsrc[2 * tid + 1]);
    __syncthreads();
    src ^= 1;
  }
  const int n_sel = min(budget, lens[src * lstride]);
  for (int o = tid; o < n_sel; o += kSelectThreads) {
    const uint32_t r = mi[src][o];
    lv_gidx[loff[r >> 16] + (r & 0xFFFFu)] = static_cast<uint16_t>(o + 1);
  }
  __syncthreads();

  // ---- phase 4: write the tree in node-index order
  const size_t base = static_cast<size_t>(seq) * (budget + 1);
  for (int o = tid; o < n_sel; o += kSelectThreads) {
    const uint32_t r = mi[src][o];
    const int d = static_cast<int>(r >> 16), i = static_cast<int>(r & 0xFFFFu);
    const int idx = loff[d] + i;
    const int g = o + 1;
    const uint32_t inf = lv_info[idx];
    const int pp = static_cast<int>(inf & 0xFFFFu), k = static_cast<int>(inf >> 16);
    parent[base + g] = (d == 1) ? 0 : static_cast<int32_t>(lv_gidx[loff[d - 1] + pp]);
    token[base + g] = ctok[(d - 1) * WMAX + k];
    depth[base + g] = d;
    if (score_out) score_out[base + g] = lv_score[idx];
  }
  for (int g = n_sel + 1 + tid; g <= budget; g += kSelectThreads) {
    parent[base + g] = -1;
    token[base + g] = -1;
    depth[base + g] = -1;
    if (score_out) score_out[base + g] = -INFINITY;
  }
  if (tid == 0) {
    parent[base] = -1;
    token[base] = root_token[seq];
    depth[base] = 0;
    if (score_out) score_out[base] = 0.0;
    n_nodes[seq] = n_sel + 1;
  }
}

// ------------------------------------------------------------------
// tree_select_seq: the build-mode variants, as a literal best-first search.
// JetSpec explainer (techwalker.com), section 五: pop the best entry of a
// priority queue, give it up to W children, repeat until B nodes are placed;
// the same section names the per-position entropy and an entropy / log-prob
// mix as alternative priorities.  With a = entropy_weight in [0, 1]:
//   key = (1 - a) * score - a * H_depth   (a == 1: key = -H_depth),
// score the cumulative draft log-probability, H_d the entropy of depth d's
// row.  expand_mode 0 (candidate): the queue holds candidates (placed node,
// rank); a pop places one node; ties by parent index, then rank.  The
// candidates of one parent are key-sorted by rank (top-W is logit-sorted), so
// each placed node keeps one head: its next unplaced rank.  expand_mode 1
// (node block): the queue holds placed nodes shallower than N; a pop attaches
// that node's W children (rank order, consecutive indices), cut at B; ties by
// node index.
// One workgroup of 256 threads per sequence; node v lives in thread v % 256,
// slot v / 256 (4 slots cover the 1024-node maximum).  Each pop is one
// workgroup argmax (wave shuffles, one barrier).
constexpr int kSeqThreads = 256;
constexpr int kSeqSlots = 1024 / kSeqThreads;
constexpr int kSeqWaves = kSeqThreads / kWave;

__device__ __forceinline__ double variant_key(double score, double ent, double a) {
#pragma clang fp contract(off)
  if (a == 1.0) return -ent;
  return (1.0 - a) * score - a * ent;
}

// (key, id) order: larger key first, then smaller id; id < 0 = empty.
__device__ __forceinline__ bool seq_better(double ka, int ia, double kb, int ib) {
  if (ia < 0) return false;
  if (ib < 0) return true;
  return ka > kb || (ka == kb && ia < ib);
}

// One step of a wave argmax over (key, id) through a DPP lane move: take the
// other lane's pair when it is better.  Lanes the move does not reach (row
// mask) keep their own pair.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_best(double& k, int& id) {
  const uint2 kb = __builtin_bit_cast(uint2, k);
  uint2 ob;
  ob.x = __builtin_amdgcn_update_dpp(kb.x, kb.x, CTRL, ROW_MASK, 0xF, false);
  ob.y = __builtin_amdgcn_update_dpp(kb.y, kb.y, CTRL, ROW_MASK, 0xF, false);
  const int oi = __builtin_amdgcn_update_dpp(id, id, CTRL, ROW_MASK, 0xF, false);
  const double ok = __builtin_bit_cast(double, ob);
  if (seq_better(ok, oi, k, id)) { k = ok; id = oi; }
}

// Wave argmax of (key, id) into lane 63: quad swaps, rotations by 4 and 8
// inside each row of 16 lanes, then row broadcasts 15 and 31 (the order is
// total, so any combination order gives the same winner).
__device__ __forceinline__ void wave_best_to_lane63(double& k, int& id) {
  dpp_best<0xB1, 0xF>(k, id);   // quad_perm [1, 0, 3, 2]
  dpp_best<0x4E, 0xF>(k, id);   // quad_perm [2, 3, 0, 1]
  dpp_best<0x124, 0xF>(k, id);  // row_ror 4
  dpp_best<0x128, 0xF>(k, id);  // row_ror 8
  dpp_best<0x142, 0xA>(k, id);  // row_bcast 15 into rows 1 and 3
  dpp_best<0x143, 0xC>(k, id);  // row_bcast 31 into rows 2 and 3
}

template <int WMAX>
__global__ __launch_bounds__(kSeqThreads) void tree_select_seq(
    const float* __restrict__ part_max, const double* __restrict__ part_sum,
    const double* __restrict__ part_ent, const float* __restrict__ part_val,
    const int* __restrict__ part_idx, int chunks, int depth_n, int width, int budget,
    int expand_mode, double a, const int32_t* __restrict__ root_token,
    int32_t* __restrict__ parent, int32_t* __restrict__ token, int32_t* __restrict__ depth,
    double* __restrict__ score_out, int32_t* __restrict__ n_nodes, int32_t* err) {
  __shared__ double lse[64], ent[64], S[65];
  __shared__ float cval[64 * WMAX];
  __shared__ int ctok[64 * WMAX];
  __shared__ double raw[1024];
  __shared__ int dep[1024];
  __shared__ double red_k[2][kSeqWaves];
  __shared__ int red_i[2][kSeqWaves];
  const int seq = blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;

  merge_depth_partials<WMAX>(part_max, part_sum, part_ent, part_val, part_idx, chunks, depth_n,
                             width, seq, lse, ent, cval, ctok, err, kSeqWaves);
  __syncthreads();
  if (tid == 0) {
    S[0] = 0.0;
    for (int d = 0; d < depth_n; ++d) S[d + 1] = S[d] + lse[d];
    raw[0] = 0.0;
    dep[0] = 0;
  }
  __syncthreads();

  const size_t base = static_cast<size_t>(seq) * (budget + 1);
  // per-slot queue entry: key and id (candidate: node << 5 | rank; block: node)
  double qk[kSeqSlots];
  int qi[kSeqSlots];
#pragma unroll
  for (int s = 0; s < kSeqSlots; ++s) { qk[s] = 0.0; qi[s] = -1; }
  // key of the candidate (u, k), u placed at depth du < depth_n
  auto cand_key = [&](int u, int du, int k) {
    const double sc = (raw[u] + static_cast<double>(cval[du * WMAX + k])) - S[du + 1];
    return variant_key(sc, ent[du], a);
  };
  if (tid == 0 && depth_n >= 1) {  // node 0 = thread 0, slot 0
    qi[0] = 0;
    qk[0] = expand_mode == 0 ? cand_key(0, 0, 0) : 0.0;
  }

  int n = 1;  // placed nodes (uniform)
  for (int pop = 0; n - 1 < budget; ++pop) {
    // ---- argmax over the queue
    double bk = 0.0;
    int bi = -1;
#pragma unroll
    for (int s = 0; s < kSeqSlots; ++s)
      if (seq_better(qk[s], qi[s], bk, bi)) { bk = qk[s]; bi = qi[s]; }
    wave_best_to_lane63(bk, bi);
    const int par = pop & 1;
    if (lane == kWave - 1) { red_k[par][wv] = bk; red_i[par][wv] = bi; }
    __syncthreads();
    bk = red_k[par][0];
    bi = red_i[par][0];
    for (int w = 1; w < kSeqWaves; ++w)
      if (seq_better(red_k[par][w], red_i[par][w], bk, bi)) { bk = red_k[par][w]; bi = red_i[par][w]; }
    if (bi < 0) break;  // queue empty (uniform)
    if (expand_mode == 0) {
      const int u = bi >> 5, k = bi & 31;
      const int du = dep[u];
      const int v = n;
      const double rv = raw[u] + static_cast<double>(cval[du * WMAX + k]);
      if (tid == u % kSeqThreads) {  // advance u's head
        const int s = u / kSeqThreads;
        if (k + 1 < width) { qi[s] = (u << 5) | (k + 1); qk[s] = cand_key(u, du, k + 1); }
        else qi[s] = -1;
      }
      if (tid == v % kSeqThreads) {  // place v, open its head
        const int s = v / kSeqThreads;
        raw[v] = rv;
        dep[v] = du + 1;
        parent[base + v] = u;
        token[base + v] = ctok[du * WMAX + k];
        depth[base + v] = du + 1;
        if (score_out) score_out[base + v] = rv - S[du + 1];
        if (du + 1 < depth_n) {
          qi[s] = v << 5;
          const double sc = (rv + static_cast<double>(cval[(du + 1) * WMAX])) - S[du + 2];
          qk[s] = variant_key(sc, ent[du + 1], a);
        }
      }
      n += 1;
    } else {
      const int u = bi;
      const int du = dep[u];
      const int c = min(width, budget - (n - 1));
      if (tid == u % kSeqThreads) qi[u / kSeqThreads] = -1;
      // child k is node v = n + k, owned by thread v % kSeqThreads: the c <= W
      // children land on distinct threads and are attached together
      const int k = (tid - n % kSeqThreads + kSeqThreads) % kSeqThreads;
      if (k < c) {
        const int v = n + k;
        const int s = v / kSeqThreads;
        const double rv = raw[u] + static_cast<double>(cval[du * WMAX + k]);
        const double sc = rv - S[du + 1];
        raw[v] = rv;
        dep[v] = du + 1;
        parent[base + v] = u;
        token[base + v] = ctok[du * WMAX + k];
        depth[base + v] = du + 1;
        if (score_out) score_out[base + v] = sc;
        if (du + 1 < depth_n) { qi[s] = v; qk[s] = variant_key(sc, ent[du], a); }
      }
      n += c;
    }
  }
  for (int g = n + tid; g <= budget; g += kSeqThreads) {
    parent[base + g] = -1;
    token[base + g] = -1;
    depth[base + g] = -1;
    if (score_out) score_out[base + g] = -INFINITY;
  }
  if (tid == 0) {
    parent[base] = -1;
    token[base] = root_token[seq];
    depth[base] = 0;
    if (score_out) score_out[base] = 0.0;
    n_nodes[seq] = n;
  }
}

// ------------------------------------------------------------------ host side

struct ScanPlan {
  int rows, chunks, chunk_len, wmax, vec, ept;
};

static int wmax_of(int width) {
  return width <= 1 ? 1 : width <= 2 ? 2 : width <= 4 ? 4 : width <= 8 ? 8 : 16;
}

// A chunk is 256 threads x EPT logits: EPT = 32 while a row fits 64 chunks,
// else 128; tree_select merges one chunk per lane.  (4K-logit chunks were
// measured slower: the per-chunk threshold and merge work dominates.)
static ScanPlan scan_plan(int batch, int depth_n, int vocab, int width, int vec) {
  ScanPlan p{};
  p.rows = batch * depth_n;
  p.vec = vec;
  p.ept = (vocab <= 64 * 256 * 32) ? 32 : 128;
  p.chunk_len = 256 * p.ept;
  p.chunks = (vocab + p.chunk_len - 1) / p.chunk_len;
  p.wmax = wmax_of(width);
  return p;
}

struct ScanWorkspace {
  size_t off_max, off_sum, off_ent, off_val, off_idx, bytes;
};

static ScanWorkspace scan_workspace(const ScanPlan& p, int width) {
  ScanWorkspace w{};
  const size_t n = static_cast<size_t>(p.rows) * p.chunks;
  size_t o = 0;
  auto take = [&](size_t b) { o = (o + 255) / 256 * 256; size_t r = o; o += b; return r; };
  w.off_max = take(n * sizeof(float));
  w.off_sum = take(n * sizeof(double));
  w.off_ent = take(n * sizeof(double));
  w.off_val = take(n * width * sizeof(float));
  w.off_idx = take(n * width * sizeof(int));
  w.bytes = (o + 255) / 256 * 256;
  return w;
}

int build_tree_max_vocab() { return 64 * 256 * 128; }

size_t build_tree_workspace_bytes(int batch, int depth_n, int vocab, int width) {
  if (batch <= 0) return 0;
  return scan_workspace(scan_plan(batch, depth_n, vocab, width, 1), width).bytes;
}

size_t build_tree_lds_bytes(int depth_n, int width, int budget) {
  return select_layout(depth_n, width, budget, wmax_of(width)).bytes;
}

struct ScanPtrs {
  float* pm;
  double* ps;
  double* pe;
  float* pv;
  int* pi;
};

template <int WMAX>
static void select_n(int batch, int depth_n, int width, int budget, const ScanPlan& p,
                     const ScanPtrs& w, const int32_t* root_token, int32_t* parent,
                     int32_t* token, int32_t* depth, double* score, int32_t* n_nodes,
                     int32_t* err, hipStream_t stream) {
  const SelectLayout L = select_layout(depth_n, width, budget, WMAX);
  if (L.bytes > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&tree_select<WMAX>),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              static_cast<int>(L.bytes));
  hipLaunchKernelGGL((tree_select<WMAX>), dim3(batch), dim3(kSelectThreads), L.bytes, stream,
                     w.pm, w.ps, w.pv, w.pi, p.chunks, depth_n, width, budget, L, root_token,
                     parent, token, depth, score, n_nodes, err);
}

template <int WMAX>
static void select_seq_n(int batch, int depth_n, int width, int budget, int expand_mode,
                         double a, const ScanPlan& p, const ScanPtrs& w,
                         const int32_t* root_token, int32_t* parent, int32_t* token,
                         int32_t* depth, double* score, int32_t* n_nodes, int32_t* err,
                         hipStream_t stream) {
  hipLaunchKernelGGL((tree_select_seq<WMAX>), dim3(batch), dim3(kSeqThreads), 0, stream, w.pm,
                     w.ps, w.pe, w.pv, w.pi, p.chunks, depth_n, width, budget, expand_mode, a,
                     root_token, parent, token, depth, score, n_nodes, err);
}

// mode < 0: the default build (tree_select); otherwise the variant search.
static hipError_t build_common(const void* logits, jt_dtype dt, int batch, int depth_n,
                               int vocab, int width, int budget, int mode, double a,
                               const int32_t* root_token, int32_t* parent, int32_t* token,
                               int32_t* depth, double* score, int32_t* n_nodes, int32_t* err,
                               void* workspace, hipStream_t stream) {
  const int vec_elems = dt == JT_F32 ? 4 : 8;
  const bool vec_ok = vocab % vec_elems == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0;
  const ScanPlan p = scan_plan(batch, depth_n, vocab, width, vec_ok ? vec_elems : 1);
  const ScanPlan p1 = scan_plan(batch, depth_n, vocab, width, 1);
  const ScanWorkspace ws_l = scan_workspace(p1, width);  // sized for the largest plan
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  const ScanPtrs w{reinterpret_cast<float*>(ws + ws_l.off_max),
                   reinterpret_cast<double*>(ws + ws_l.off_sum),
                   reinterpret_cast<double*>(ws + ws_l.off_ent),
                   reinterpret_cast<float*>(ws + ws_l.off_val),
                   reinterpret_cast<int*>(ws + ws_l.off_idx)};
  const ScanArgs sa{p.rows, p.chunks, p.chunk_len, p.ept, p.vec, p.wmax,
                    w.pm, w.ps, w.pe, w.pv, w.pi, err};
  hipError_t e = draft_scan_launch(logits, dt, mode >= 0, vocab, width, sa, stream);
  if (e != hipSuccess) return e;
#define JT_SELECT(WM)                                                                       \
  if (mode < 0)                                                                             \
    select_n<WM>(batch, depth_n, width, budget, p, w, root_token, parent, token, depth, score, \
                 n_nodes, err, stream);                                                     \
  else                                                                                      \
    select_seq_n<WM>(batch, depth_n, width, budget, mode, a, p, w, root_token, parent, token, \
                     depth, score, n_nodes, err, stream)
  switch (p.wmax) {
    case 1: JT_SELECT(1); break;
    case 2: JT_SELECT(2); break;
    case 4: JT_SELECT(4); break;
    case 8: JT_SELECT(8); break;
    default: JT_SELECT(16); break;
  }
#undef JT_SELECT
  return hipGetLastError();
}

hipError_t build_tree_launch(const void* logits, jt_dtype dt, int batch, int depth_n, int vocab,
                             int width, int budget, const int32_t* root_token, int32_t* parent,
                             int32_t* token, int32_t* depth, double* score, int32_t* n_nodes,
                             int32_t* err, void* workspace, hipStream_t stream) {
  return build_common(logits, dt, batch, depth_n, vocab, width, budget, -1, 0.0, root_token,
                      parent, token, depth, score, n_nodes, err, workspace, stream);
}

hipError_t build_tree_variant_launch(const void* logits, jt_dtype dt, int batch, int depth_n,
                                     int vocab, int width, int budget, int expand_mode,
                                     double entropy_weight, const int32_t* root_token,
                                     int32_t* parent, int32_t* token, int32_t* depth,
                                     double* score, int32_t* n_nodes, int32_t* err,
                                     void* workspace, hipStream_t stream) {
  return build_common(logits, dt, batch, depth_n, vocab, width, budget, expand_mode,
                      entropy_weight, root_token, parent, token, depth, score, n_nodes, err,
                      workspace, stream);
}

}  // namespace jt
