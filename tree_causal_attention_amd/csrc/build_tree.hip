// jt_build_tree: per-depth log-sum-exp + top-W (draft_row_scan), then the
// best-first selection of the tree (tree_select).
//
// Method: JetSpec news piece (mlqm.cn/news/158889), tree-construction
// paragraph; JetSpec explainer (techwalker.com, "加速AI思考…"), section 五.
//
// draft_row_scan: one workgroup per (vocab chunk, depth row); reads the logits
//   with 16-byte loads, finds the chunk max and per-thread sorted top-W lists,
//   then sums exp(x - max) in fp64 over the (L2-resident) chunk and merges the
//   lists over the workgroup.
// tree_select: one workgroup per sequence.  The best-first pop order equals
//   the B smallest keys (-score, parent index, rank) of the complete tree,
//   because a child never precedes its parent.  It is computed level by level:
//   level d keeps the best cap_d = min(W^d, B-d+1) children of level d-1 (a
//   depth-d node in the final tree is preceded by its d-1 ancestors, so no
//   deeper position can be selected), ranked by counting with binary searches
//   in the sorted W x m candidate matrix; then every kept node gets its global
//   rank by binary search in the other levels.  All arithmetic on scores is
//   fp64 and identical to a sequential evaluation except the per-depth
//   log-sum-exp, whose summation order differs.
#include "jt_device.h"
#include "jt_host.h"

#include <algorithm>
#include <cmath>

namespace jt {

constexpr int kScanThreads = 256;
constexpr int kSelectThreads = 1024;

template <typename T, int VEC>
__device__ __forceinline__ void load_vec(const T* x, int i, float (&v)[VEC]) {
  if constexpr (VEC == 1) {
    v[0] = load_as_f32(x, i);
  } else if constexpr (sizeof(T) == 4) {
    const float4 f = *reinterpret_cast<const float4*>(x + i);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  } else {
    const uint4 u = *reinterpret_cast<const uint4*>(x + i);
    const uint32_t wds[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(wds[k] << 16);
      v[2 * k + 1] = __uint_as_float(wds[k] & 0xFFFF0000u);
    }
  }
}

constexpr int kCandCap = 1024;  // threshold candidates kept per chunk

// One workgroup per (vocab chunk, depth row); thread t holds EPT logits of
// the chunk in registers (16-byte loads, one pass over HBM).
//  * max and the fp64 sum of exp(x - max) come straight from the registers;
//  * top-W: the W-th largest per-thread maximum L is a lower bound of the
//    chunk's W-th largest logit (W distinct threads hold a value >= L), so
//    only logits >= L are collected in LDS and ranked; if more than kCandCap
//    qualify (e.g. massive ties) every thread builds its exact sorted top-W and
//    W rounds of "best head" merge them.
template <typename T, int WMAX, int VEC, int EPT>
__global__ __launch_bounds__(kScanThreads) void draft_row_scan(
    const T* __restrict__ logits, int vocab, int chunks, int chunk_len, int width,
    float* __restrict__ part_max, double* __restrict__ part_sum, float* __restrict__ part_val,
    int* __restrict__ part_idx, int32_t* err) {
  constexpr int NV = EPT / VEC;
  __shared__ float sm_m[kScanThreads / kWave];
  __shared__ double sm_s[kScanThreads / kWave];
  __shared__ float sm_tmax[kScanThreads];
  __shared__ float sm_cv[kCandCap];
  __shared__ int sm_ci[kCandCap];
  __shared__ int sm_n;
  __shared__ float sm_L;
  __shared__ float sm_v[kScanThreads / kWave];
  __shared__ int sm_i[kScanThreads / kWave];

  const int row = blockIdx.y, c = blockIdx.x, t = threadIdx.x;
  const int lane = t % kWave, wv = t / kWave;
  const int begin = c * chunk_len;
  const int end = min(vocab, begin + chunk_len);
  const T* x = logits + static_cast<size_t>(row) * vocab;

  float xv[EPT];
  bool bad = false;
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = begin + (j * kScanThreads + t) * VEC;
    float v[VEC];
    if (i < end) {
      load_vec<T, VEC>(x, i, v);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) v[e] = -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      float y = v[e];
      if (y != y || y == INFINITY) { bad = true; y = -INFINITY; }
      xv[j * VEC + e] = y;
      m = fmaxf(m, y);
    }
  }
  if (bad) report(err, JT_DERR_BAD_LOGIT);
  if (t == 0) sm_n = 0;

  // ---- chunk max
  float wm = m;
  for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, shfl_xor(wm, o));
  if (lane == 0) sm_m[wv] = wm;
  sm_tmax[t] = m;
  __syncthreads();
  float M = sm_m[0];
  for (int w = 1; w < kScanThreads / kWave; ++w) M = fmaxf(M, sm_m[w]);

  // ---- fp64 sum of exp(x - M) over the registers
  double sacc = 0.0;
  if (M != -INFINITY) {
    const double Md = static_cast<double>(M);
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const double e = exp(static_cast<double>(fmaxf(xv[k], -1.0e30f)) - Md);
      sacc += (xv[k] != -INFINITY) ? e : 0.0;
    }
  }
  for (int o = 32; o > 0; o >>= 1) sacc += shfl_xor_f64(sacc, o);
  if (lane == 0) sm_s[wv] = sacc;

  // ---- threshold: the W-th largest thread maximum (ties by thread id)
  int rank = 0;
  for (int u = 0; u < kScanThreads; ++u) {
    const float mu = sm_tmax[u];
    rank += (mu > m || (mu == m && u < t)) ? 1 : 0;
  }
  if (rank == width - 1) sm_L = m;
  __syncthreads();
  if (t == 0) {
    double S = 0.0;
    for (int w = 0; w < kScanThreads / kWave; ++w) S += sm_s[w];
    part_max[row * chunks + c] = M;
    part_sum[row * chunks + c] = S;
  }
  const float L = sm_L;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = begin + (j * kScanThreads + t) * VEC;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (i + e < end && xv[j * VEC + e] >= L) {
        const int pos = atomicAdd(&sm_n, 1);
        if (pos < kCandCap) { sm_cv[pos] = xv[j * VEC + e]; sm_ci[pos] = i + e; }
      }
    }
  }
  __syncthreads();
  const int nc = sm_n;
  const size_t out0 = (static_cast<size_t>(row) * chunks + c) * width;
  if (nc <= kCandCap) {
    for (int q = t; q < nc; q += kScanThreads) {
      const float vq = sm_cv[q];
      const int iq = sm_ci[q];
      int r = 0;
      for (int u = 0; u < nc; ++u) r += better(sm_cv[u], sm_ci[u], vq, iq) ? 1 : 0;
      if (r < width) { part_val[out0 + r] = vq; part_idx[out0 + r] = iq; }
    }
    for (int r = nc + t; r < width; r += kScanThreads) {
      part_val[out0 + r] = -INFINITY;
      part_idx[out0 + r] = INT32_MAX;
    }
    return;
  }

  // ---- overflow: exact per-thread sorted lists, merged by W rounds
  float tv[WMAX];
  int ti[WMAX];
#pragma unroll
  for (int k = 0; k < WMAX; ++k) { tv[k] = -INFINITY; ti[k] = INT32_MAX; }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int i = begin + (j * kScanThreads + t) * VEC + e;
      const float y = xv[j * VEC + e];
      if (i < end && better(y, i, tv[WMAX - 1], ti[WMAX - 1])) {
        // Sorted insert as a select network: slot k keeps its entry if it
        // precedes the new one, takes the new one at the first slot it beats,
        // and takes its predecessor's entry after that.  Slots are rewritten
        // from the last one up, so slot k-1 still holds its old entry.
#pragma unroll
        for (int k = WMAX - 1; k >= 0; --k) {
          const int u = k > 0 ? k - 1 : 0;
          const bool b = better(y, i, tv[k], ti[k]);
          const bool b_up = k > 0 && better(y, i, tv[u], ti[u]);
          const float up_v = tv[u];
          const int up_i = ti[u];
          tv[k] = b ? (b_up ? up_v : y) : tv[k];
          ti[k] = b ? (b_up ? up_i : i) : ti[k];
        }
      }
    }
  }
  for (int r = 0; r < width; ++r) {
    float bv = tv[0];
    int bi = ti[0];
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = shfl_xor(bv, o);
      const int oi = shfl_xor(bi, o);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    __syncthreads();  // previous round's readers are done with sm_v/sm_i
    if (lane == 0) { sm_v[wv] = bv; sm_i[wv] = bi; }
    __syncthreads();
    float gv = sm_v[0];
    int gi = sm_i[0];
    for (int w = 1; w < kScanThreads / kWave; ++w)
      if (better(sm_v[w], sm_i[w], gv, gi)) { gv = sm_v[w]; gi = sm_i[w]; }
    if (t == 0) { part_val[out0 + r] = gv; part_idx[out0 + r] = gi; }
    if (ti[0] == gi && gi != INT32_MAX) {
#pragma unroll
      for (int k = 0; k + 1 < WMAX; ++k) { tv[k] = tv[k + 1]; ti[k] = ti[k + 1]; }
      tv[WMAX - 1] = -INFINITY;
      ti[WMAX - 1] = INT32_MAX;
    }
  }
}

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
  int top;         // power of two >= capmax (binary-lifting start)
  size_t off_S, off_lse, off_cval, off_ctok, off_loff, off_lcnt, off_rawa, off_rawb;
  size_t off_score, off_info, off_gidx, bytes;
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
  L.top = 1;
  while (L.top < L.capmax) L.top <<= 1;
  size_t o = 0;
  auto take = [&](size_t n, size_t align) { o = (o + align - 1) / align * align; size_t r = o; o += n; return r; };
  L.off_S = take(sizeof(double) * (depth_n + 1), 8);
  L.off_lse = take(sizeof(double) * depth_n, 8);
  L.off_rawa = take(sizeof(double) * L.capmax, 8);
  L.off_rawb = take(sizeof(double) * L.capmax, 8);
  L.off_score = take(sizeof(double) * std::max(1, L.tot), 8);
  L.off_cval = take(sizeof(float) * depth_n * wmax, 4);
  L.off_ctok = take(sizeof(int) * depth_n * wmax, 4);
  L.off_loff = take(sizeof(int) * (depth_n + 2), 4);
  L.off_lcnt = take(sizeof(int) * (depth_n + 2), 4);
  L.off_info = take(sizeof(uint32_t) * std::max(1, L.tot), 4);
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

// Binary lifting over a prefix-true predicate runs a fixed number of steps
// (top = a power of two >= every list length), so the W - 1 (or N - 1)
// searches of one candidate advance in lockstep and their LDS reads overlap.
template <int WMAX, int NMAX>
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
  float* cval = reinterpret_cast<float*>(smem + L.off_cval);
  int* ctok = reinterpret_cast<int*>(smem + L.off_ctok);
  int* loff = reinterpret_cast<int*>(smem + L.off_loff);
  int* lcnt = reinterpret_cast<int*>(smem + L.off_lcnt);
  uint32_t* lv_info = reinterpret_cast<uint32_t*>(smem + L.off_info);
  uint16_t* lv_gidx = reinterpret_cast<uint16_t*>(smem + L.off_gidx);

  const int seq = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int nwaves = kSelectThreads / kWave;
  const int top = L.top;

  // ---- phase 1: merge the chunk partials of every depth (one wave a depth);
  // each lane holds one chunk's sorted candidates in registers.
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
    double contrib = (mc == -INFINITY) ? 0.0 : sc * exp(static_cast<double>(mc) - static_cast<double>(M));
    for (int o = 32; o > 0; o >>= 1) contrib += shfl_xor_f64(contrib, o);
    if (lane == 0) {
      if (M == -INFINITY) {
        report(err, JT_DERR_BAD_LOGIT);
        lse[d] = 0.0;
      } else {
        lse[d] = static_cast<double>(M) + log(contrib);
      }
    }
    for (int r = 0; r < width; ++r) {
      float bv = hv[0];
      int bi = hid[0];
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = shfl_xor(bv, o);
        const int oi = shfl_xor(bi, o);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (hid[0] == bi && bi != INT32_MAX) {  // this lane's head won: pop it
#pragma unroll
        for (int k = 0; k + 1 < WMAX; ++k) { hv[k] = hv[k + 1]; hid[k] = hid[k + 1]; }
        hv[WMAX - 1] = -INFINITY;
        hid[WMAX - 1] = INT32_MAX;
      }
      if (lane == 0) { cval[d * WMAX + r] = bv; ctok[d * WMAX + r] = bi; }
    }
  }
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
  __syncthreads();

  // ---- phase 2: level by level, keep the best cap_d children, in order
  double* raw_prev = raw_a;
  double* raw_cur = raw_b;
  int m_prev = 1;
  int last_level = 0;
  for (int d = 1; d <= depth_n; ++d) {
    const int cap = level_cap(d, width, budget);
    if (cap <= 0 || m_prev == 0) break;
    const double Sd = S[d];
    double cv[WMAX];
#pragma unroll
    for (int k = 0; k < WMAX; ++k) cv[k] = static_cast<double>(cval[(d - 1) * WMAX + (k < width ? k : 0)]);
    const int ncand = m_prev * width;
    for (int idx = tid; idx < ncand; idx += kSelectThreads) {
      const int k = idx / m_prev, p = idx % m_prev;
      if ((p + 1) * (k + 1) > cap) continue;
      double vk = cv[0];
#pragma unroll
      for (int kk = 1; kk < WMAX; ++kk) vk = (kk == k) ? cv[kk] : vk;
      const double raw = raw_prev[p] + vk;
      const double sc = raw - Sd;
      int cnt[WMAX];
#pragma unroll
      for (int k2 = 0; k2 < WMAX; ++k2) cnt[k2] = 0;
      for (int sz = top; sz > 0; sz >>= 1) {
        // branch-free step: every column's read is issued before any compare
#pragma unroll
        for (int k2 = 0; k2 < WMAX; ++k2) {
          const int mid = cnt[k2] + sz;
          const int q = min(mid, m_prev) - 1;
          const double s2 = (raw_prev[q] + cv[k2]) - Sd;
          const bool pred = k2 < width && k2 != k && mid <= m_prev &&
                            (s2 > sc || (s2 == sc && (k2 < k ? q <= p : q < p)));
          cnt[k2] = pred ? mid : cnt[k2];
        }
      }
      int r = p;
#pragma unroll
      for (int k2 = 0; k2 < WMAX; ++k2) r += cnt[k2];
      if (r < cap) {
        lv_score[loff[d] + r] = sc;
        lv_info[loff[d] + r] = static_cast<uint32_t>(p) | (static_cast<uint32_t>(k) << 16);
        raw_cur[r] = raw;
      }
    }
    const int m_d = min(cap, ncand);
    if (tid == 0) lcnt[d] = m_d;
    __syncthreads();
    double* t = raw_prev; raw_prev = raw_cur; raw_cur = t;
    m_prev = m_d;
    last_level = d;
  }
  if (tid == 0)
    for (int d = last_level + 1; d <= depth_n; ++d) lcnt[d] = 0;
  __syncthreads();

  // ---- phase 3: global rank of every kept node (lockstep searches over levels)
  int lo_r[NMAX], lc_r[NMAX];
  int total = 0;
#pragma unroll
  for (int d2 = 0; d2 < NMAX; ++d2) {
    lo_r[d2] = (d2 + 1 <= depth_n) ? loff[d2 + 1] : 0;
    lc_r[d2] = (d2 + 1 <= depth_n) ? lcnt[d2 + 1] : 0;
    total += lc_r[d2];
  }
  const int n_sel = min(budget, total);
  for (int idx = tid; idx < loff[depth_n + 1]; idx += kSelectThreads) {
    int d = 1;
    while (idx >= loff[d + 1]) ++d;
    const int i = idx - loff[d];
    if (i >= lcnt[d]) continue;
    const double sx = lv_score[idx];
    int cnt[NMAX];
#pragma unroll
    for (int d2 = 0; d2 < NMAX; ++d2) cnt[d2] = 0;
    for (int sz = top; sz > 0; sz >>= 1) {
      // fast path branch-free; exact cross-level score ties (rare) resolved after
      bool tie[NMAX];
      bool any_tie = false;
#pragma unroll
      for (int d2 = 0; d2 < NMAX; ++d2) {
        const int mid = cnt[d2] + sz;
        const bool ok = d2 + 1 != d && mid <= lc_r[d2];
        const int q = max(0, min(mid, lc_r[d2]) - 1);
        const double sy = lv_score[lo_r[d2] + q];
        tie[d2] = ok && sy == sx;
        any_tie |= tie[d2];
        cnt[d2] = (ok && sy > sx) ? mid : cnt[d2];
      }
      if (any_tie) {
#pragma unroll
        for (int d2 = 0; d2 < NMAX; ++d2)
          if (tie[d2] && precedes_tied(lv_score, lv_info, loff, d2 + 1, cnt[d2] + sz - 1, d, i))
            cnt[d2] += sz;
      }
    }
    int R = i;
#pragma unroll
    for (int d2 = 0; d2 < NMAX; ++d2) R += cnt[d2];
    lv_gidx[idx] = (R < budget) ? static_cast<uint16_t>(R + 1) : static_cast<uint16_t>(0xFFFF);
  }
  __syncthreads();

  // ---- phase 4: write the tree in node-index order
  const size_t base = static_cast<size_t>(seq) * (budget + 1);
  for (int idx = tid; idx < loff[depth_n + 1]; idx += kSelectThreads) {
    int d = 1;
    while (idx >= loff[d + 1]) ++d;
    const int i = idx - loff[d];
    if (i >= lcnt[d]) continue;
    const int g = lv_gidx[idx];
    if (g == 0xFFFF) continue;
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

// ------------------------------------------------------------------ host side

struct ScanPlan {
  int rows, chunks, chunk_len, wmax, vec, ept;
};

static int wmax_of(int width) {
  return width <= 1 ? 1 : width <= 2 ? 2 : width <= 4 ? 4 : width <= 8 ? 8 : 16;
}

// A chunk is 256 threads x EPT logits (EPT = 32, or 128 for vocabularies
// past 512K); at most 64 chunks per row (tree_select merges one per lane).
static ScanPlan scan_plan(int batch, int depth_n, int vocab, int width, int vec) {
  ScanPlan p{};
  p.rows = batch * depth_n;
  p.vec = vec;
  p.ept = (vocab <= 64 * kScanThreads * 32) ? 32 : 128;
  p.chunk_len = kScanThreads * p.ept;
  p.chunks = (vocab + p.chunk_len - 1) / p.chunk_len;
  p.wmax = wmax_of(width);
  return p;
}

struct ScanWorkspace {
  size_t off_max, off_sum, off_val, off_idx, bytes;
};

static ScanWorkspace scan_workspace(const ScanPlan& p, int width) {
  ScanWorkspace w{};
  const size_t n = static_cast<size_t>(p.rows) * p.chunks;
  size_t o = 0;
  auto take = [&](size_t b) { o = (o + 255) / 256 * 256; size_t r = o; o += b; return r; };
  w.off_max = take(n * sizeof(float));
  w.off_sum = take(n * sizeof(double));
  w.off_val = take(n * width * sizeof(float));
  w.off_idx = take(n * width * sizeof(int));
  w.bytes = (o + 255) / 256 * 256;
  return w;
}

int build_tree_max_vocab() { return 64 * kScanThreads * 128; }

size_t build_tree_workspace_bytes(int batch, int depth_n, int vocab, int width) {
  if (batch <= 0) return 0;
  // vec 1 gives the most chunks of the possible plans
  return scan_workspace(scan_plan(batch, depth_n, vocab, width, 1), width).bytes;
}

size_t build_tree_lds_bytes(int depth_n, int width, int budget) {
  return select_layout(depth_n, width, budget, wmax_of(width)).bytes;
}

template <typename T, int WMAX, int VEC>
static void launch_scan(const void* logits, int vocab, int width, const ScanPlan& p, float* pm,
                        double* ps, float* pv, int* pi, int32_t* err, hipStream_t stream) {
  if (p.ept == 32)
    hipLaunchKernelGGL((draft_row_scan<T, WMAX, VEC, 32>), dim3(p.chunks, p.rows),
                       dim3(kScanThreads), 0, stream, static_cast<const T*>(logits), vocab,
                       p.chunks, p.chunk_len, width, pm, ps, pv, pi, err);
  else
    hipLaunchKernelGGL((draft_row_scan<T, WMAX, VEC, 128>), dim3(p.chunks, p.rows),
                       dim3(kScanThreads), 0, stream, static_cast<const T*>(logits), vocab,
                       p.chunks, p.chunk_len, width, pm, ps, pv, pi, err);
}

template <typename T, int WMAX>
static void scan_vec(const void* logits, int vocab, int width, const ScanPlan& p, float* pm,
                     double* ps, float* pv, int* pi, int32_t* err, hipStream_t stream) {
  constexpr int V = sizeof(T) == 4 ? 4 : 8;
  if (p.vec == V) launch_scan<T, WMAX, V>(logits, vocab, width, p, pm, ps, pv, pi, err, stream);
  else launch_scan<T, WMAX, 1>(logits, vocab, width, p, pm, ps, pv, pi, err, stream);
}

template <typename T>
static void scan_w(const void* logits, int vocab, int width, const ScanPlan& p, float* pm,
                   double* ps, float* pv, int* pi, int32_t* err, hipStream_t stream) {
  switch (p.wmax) {
    case 1: scan_vec<T, 1>(logits, vocab, width, p, pm, ps, pv, pi, err, stream); break;
    case 2: scan_vec<T, 2>(logits, vocab, width, p, pm, ps, pv, pi, err, stream); break;
    case 4: scan_vec<T, 4>(logits, vocab, width, p, pm, ps, pv, pi, err, stream); break;
    case 8: scan_vec<T, 8>(logits, vocab, width, p, pm, ps, pv, pi, err, stream); break;
    default: scan_vec<T, 16>(logits, vocab, width, p, pm, ps, pv, pi, err, stream); break;
  }
}

template <int WMAX>
static void select_n(int batch, int depth_n, int width, int budget, const ScanPlan& p,
                     const float* pm, const double* ps, const float* pv, const int* pi,
                     const int32_t* root_token, int32_t* parent, int32_t* token, int32_t* depth,
                     double* score, int32_t* n_nodes, int32_t* err, hipStream_t stream) {
  const SelectLayout L = select_layout(depth_n, width, budget, WMAX);
  if (depth_n <= 16)
    hipLaunchKernelGGL((tree_select<WMAX, 16>), dim3(batch), dim3(kSelectThreads), L.bytes, stream,
                       pm, ps, pv, pi, p.chunks, depth_n, width, budget, L, root_token, parent,
                       token, depth, score, n_nodes, err);
  else
    hipLaunchKernelGGL((tree_select<WMAX, 64>), dim3(batch), dim3(kSelectThreads), L.bytes, stream,
                       pm, ps, pv, pi, p.chunks, depth_n, width, budget, L, root_token, parent,
                       token, depth, score, n_nodes, err);
}

hipError_t build_tree_launch(const void* logits, jt_dtype dt, int batch, int depth_n, int vocab,
                             int width, int budget, const int32_t* root_token, int32_t* parent,
                             int32_t* token, int32_t* depth, double* score, int32_t* n_nodes,
                             int32_t* err, void* workspace, hipStream_t stream) {
  const int vec_elems = dt == JT_F32 ? 4 : 8;
  const bool vec_ok = vocab % vec_elems == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0;
  const ScanPlan p = scan_plan(batch, depth_n, vocab, width, vec_ok ? vec_elems : 1);
  const ScanPlan p1 = scan_plan(batch, depth_n, vocab, width, 1);
  const ScanWorkspace w = scan_workspace(p1, width);  // sized for the largest plan
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  float* pm = reinterpret_cast<float*>(ws + w.off_max);
  double* ps = reinterpret_cast<double*>(ws + w.off_sum);
  float* pv = reinterpret_cast<float*>(ws + w.off_val);
  int* pi = reinterpret_cast<int*>(ws + w.off_idx);
  if (dt == JT_F32) scan_w<float>(logits, vocab, width, p, pm, ps, pv, pi, err, stream);
  else scan_w<uint16_t>(logits, vocab, width, p, pm, ps, pv, pi, err, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (p.wmax) {
    case 1: select_n<1>(batch, depth_n, width, budget, p, pm, ps, pv, pi, root_token, parent, token, depth, score, n_nodes, err, stream); break;
    case 2: select_n<2>(batch, depth_n, width, budget, p, pm, ps, pv, pi, root_token, parent, token, depth, score, n_nodes, err, stream); break;
    case 4: select_n<4>(batch, depth_n, width, budget, p, pm, ps, pv, pi, root_token, parent, token, depth, score, n_nodes, err, stream); break;
    case 8: select_n<8>(batch, depth_n, width, budget, p, pm, ps, pv, pi, root_token, parent, token, depth, score, n_nodes, err, stream); break;
    default: select_n<16>(batch, depth_n, width, budget, p, pm, ps, pv, pi, root_token, parent, token, depth, score, n_nodes, err, stream); break;
  }
  return hipGetLastError();
}

}  // namespace jt
