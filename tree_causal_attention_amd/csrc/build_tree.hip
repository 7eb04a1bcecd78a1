// jt_build_tree: per-depth log-sum-exp + top-W (draft_row_scan), then the
// best-first selection of the tree (tree_select).
//
// Method: JetSpec news piece (mlqm.cn/news/158889), tree-construction
// paragraph; JetSpec explainer (techwalker.com, "加速AI思考…"), section 五.
//
// draft_row_scan: one workgroup per (row chunk, depth row); streams the fp32
//   logits once, keeping a running (max, fp64 sum of exp) and a per-thread
//   sorted top-W list, then reduces them over the workgroup.  HBM-bound.
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

template <typename T, int WMAX>
__global__ __launch_bounds__(kScanThreads) void draft_row_scan(
    const T* __restrict__ logits, int vocab, int chunks, int chunk_len, int width,
    float* __restrict__ part_max, double* __restrict__ part_sum, float* __restrict__ part_val,
    int* __restrict__ part_idx, int32_t* err) {
  const int row = blockIdx.y, c = blockIdx.x;
  const int begin = c * chunk_len;
  const int end = min(vocab, begin + chunk_len);
  const T* x = logits + static_cast<size_t>(row) * vocab;

  float m = -INFINITY;
  double s = 0.0;
  bool bad = false;
  float tv[WMAX];
  int ti[WMAX];
#pragma unroll
  for (int k = 0; k < WMAX; ++k) { tv[k] = -INFINITY; ti[k] = INT32_MAX; }

  for (int i = begin + threadIdx.x; i < end; i += kScanThreads) {
    const float v = load_as_f32(x, i);
    if (v != v || v == INFINITY) { bad = true; continue; }
    if (v != -INFINITY) {
      if (v > m) {
        s = s * exp(static_cast<double>(m) - static_cast<double>(v)) + 1.0;
        m = v;
      } else {
        s += exp(static_cast<double>(v) - static_cast<double>(m));
      }
    }
    if (better(v, i, tv[WMAX - 1], ti[WMAX - 1])) {
      // Sorted insert as a select network: slot k keeps its entry if it
      // precedes the new one, takes the new one at the first slot it beats,
      // and takes its predecessor's entry after that.  Slots are rewritten
      // from the last one up, so slot k-1 still holds its old entry.
#pragma unroll
      for (int k = WMAX - 1; k >= 0; --k) {
        const int u = k > 0 ? k - 1 : 0;
        const bool b = better(v, i, tv[k], ti[k]);
        const bool b_up = k > 0 && better(v, i, tv[u], ti[u]);
        const float up_v = tv[u];
        const int up_i = ti[u];
        tv[k] = b ? (b_up ? up_v : v) : tv[k];
        ti[k] = b ? (b_up ? up_i : i) : ti[k];
      }
    }
  }
  if (bad) report(err, JT_DERR_BAD_LOGIT);

  // ---- (max, sum) over the workgroup
  __shared__ float sm_m[kScanThreads / kWave];
  __shared__ double sm_s[kScanThreads / kWave];
  __shared__ float sm_v[kScanThreads / kWave];
  __shared__ int sm_i[kScanThreads / kWave];
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  float wm = m;
  for (int o = 32; o > 0; o >>= 1) wm = fmaxf(wm, shfl_xor(wm, o));
  double ws = (m == -INFINITY) ? 0.0 : s * exp(static_cast<double>(m) - static_cast<double>(wm));
  for (int o = 32; o > 0; o >>= 1) ws += shfl_xor_f64(ws, o);
  if (lane == 0) { sm_m[wv] = wm; sm_s[wv] = ws; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = -INFINITY;
    for (int w = 0; w < kScanThreads / kWave; ++w) M = fmaxf(M, sm_m[w]);
    double S = 0.0;
    for (int w = 0; w < kScanThreads / kWave; ++w)
      if (sm_m[w] != -INFINITY) S += sm_s[w] * exp(static_cast<double>(sm_m[w]) - static_cast<double>(M));
    part_max[row * chunks + c] = M;
    part_sum[row * chunks + c] = S;
  }

  // ---- top-W over the workgroup: W rounds of (best head, pop it)
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
    if (threadIdx.x == 0) {
      part_val[(static_cast<size_t>(row) * chunks + c) * width + r] = gv;
      part_idx[(static_cast<size_t>(row) * chunks + c) * width + r] = gi;
    }
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

// Number of candidates (p', k2) of the level being built that precede the
// candidate with score s and parent position p: the predicate is true on a
// prefix of p' because column k2 is sorted by score.
__device__ __forceinline__ int count_before(const double* raw_prev, int m, double vk2, double Sd,
                                            double s, int p, bool inclusive) {
  int lo = 0, hi = m;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const double sc = (raw_prev[mid] + vk2) - Sd;
    const bool pred = sc > s || (sc == s && (inclusive ? mid <= p : mid < p));
    if (pred) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Does kept node (d2, j) precede kept node (d, i), d2 != d?  Scores first;
// exact ties compare the parents' keys, walking up both paths (their depths
// keep differing, so they never meet; the root precedes every other node).
__device__ __forceinline__ bool precedes_cross(const double* score, const uint32_t* info,
                                               const int* loff, int d2, int j, int d, int i) {
  while (true) {
    const double sy = score[loff[d2] + j];
    const double sx = score[loff[d] + i];
    if (sy != sx) return sy > sx;
    j = static_cast<int>(info[loff[d2] + j] & 0xFFFFu);
    i = static_cast<int>(info[loff[d] + i] & 0xFFFFu);
    --d2;
    --d;
    if (d2 == 0) return true;
    if (d == 0) return false;
  }
}

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
  float* cval = reinterpret_cast<float*>(smem + L.off_cval);
  int* ctok = reinterpret_cast<int*>(smem + L.off_ctok);
  int* loff = reinterpret_cast<int*>(smem + L.off_loff);
  int* lcnt = reinterpret_cast<int*>(smem + L.off_lcnt);
  uint32_t* lv_info = reinterpret_cast<uint32_t*>(smem + L.off_info);
  uint16_t* lv_gidx = reinterpret_cast<uint16_t*>(smem + L.off_gidx);

  const int seq = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int nwaves = kSelectThreads / kWave;

  // ---- phase 1: merge the chunk partials of every depth (one wave a depth)
  for (int d = wv; d < depth_n; d += nwaves) {
    const size_t row = static_cast<size_t>(seq) * depth_n + d;
    const bool act = lane < chunks;
    const float mc = act ? part_max[row * chunks + lane] : -INFINITY;
    const double sc = act ? part_sum[row * chunks + lane] : 0.0;
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
    int ptr = 0;
    for (int r = 0; r < width; ++r) {
      float hv = -INFINITY;
      int hi = INT32_MAX;
      if (act && ptr < width) {
        hv = part_val[(row * chunks + lane) * width + ptr];
        hi = part_idx[(row * chunks + lane) * width + ptr];
      }
      float bv = hv;
      int bi = hi;
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = shfl_xor(bv, o);
        const int oi = shfl_xor(bi, o);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      if (act && ptr < width && hi == bi) ++ptr;
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
    const int ncand = m_prev * width;
    for (int idx = tid; idx < ncand; idx += kSelectThreads) {
      const int k = idx / m_prev, p = idx % m_prev;
      if ((p + 1) * (k + 1) > cap) continue;
      const double vk = static_cast<double>(cval[(d - 1) * WMAX + k]);
      const double raw = raw_prev[p] + vk;
      const double s = raw - Sd;
      int r = p;
      for (int k2 = 0; k2 < width; ++k2) {
        if (k2 == k) continue;
        r += count_before(raw_prev, m_prev, static_cast<double>(cval[(d - 1) * WMAX + k2]), Sd, s, p,
                          k2 < k);
        if (r >= cap) break;
      }
      if (r < cap) {
        lv_score[loff[d] + r] = s;
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

  // ---- phase 3: global rank of every kept node
  int total = 0;
  for (int d = 1; d <= depth_n; ++d) total += lcnt[d];
  const int n_sel = min(budget, total);
  for (int idx = tid; idx < loff[depth_n + 1]; idx += kSelectThreads) {
    int d = 1;
    while (idx >= loff[d + 1]) ++d;
    const int i = idx - loff[d];
    if (i >= lcnt[d]) continue;
    int R = i;
    for (int d2 = 1; d2 <= depth_n && R < budget; ++d2) {
      if (d2 == d || lcnt[d2] == 0) continue;
      int lo = 0, hi = lcnt[d2];
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (precedes_cross(lv_score, lv_info, loff, d2, mid, d, i)) lo = mid + 1; else hi = mid;
      }
      R += lo;
    }
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
  int rows, chunks, chunk_len, wmax;
};

static ScanPlan scan_plan(int batch, int depth_n, int vocab, int width) {
  ScanPlan p{};
  p.rows = batch * depth_n;
  const int by_rows = std::max(1, (1024 + p.rows - 1) / std::max(1, p.rows));
  const int by_vocab = std::max(1, (vocab + 2047) / 2048);
  p.chunks = std::min(64, std::min(by_rows, by_vocab));
  p.chunk_len = (vocab + p.chunks - 1) / p.chunks;
  p.chunks = (vocab + p.chunk_len - 1) / p.chunk_len;
  p.wmax = width <= 1 ? 1 : width <= 2 ? 2 : width <= 4 ? 4 : width <= 8 ? 8 : 16;
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

size_t build_tree_workspace_bytes(int batch, int depth_n, int vocab, int width) {
  if (batch <= 0) return 0;
  return scan_workspace(scan_plan(batch, depth_n, vocab, width), width).bytes;
}

size_t build_tree_lds_bytes(int depth_n, int width, int budget) {
  const ScanPlan p = scan_plan(1, depth_n, std::max(width, 1), width);
  return select_layout(depth_n, width, budget, p.wmax).bytes;
}

template <typename T, int WMAX>
static hipError_t launch_build(const void* logits, int batch, int depth_n, int vocab, int width,
                               int budget, const ScanPlan& p, const ScanWorkspace& w,
                               unsigned char* ws, const int32_t* root_token, int32_t* parent,
                               int32_t* token, int32_t* depth, double* score, int32_t* n_nodes,
                               int32_t* err, hipStream_t stream) {
  float* part_max = reinterpret_cast<float*>(ws + w.off_max);
  double* part_sum = reinterpret_cast<double*>(ws + w.off_sum);
  float* part_val = reinterpret_cast<float*>(ws + w.off_val);
  int* part_idx = reinterpret_cast<int*>(ws + w.off_idx);
  hipLaunchKernelGGL((draft_row_scan<T, WMAX>), dim3(p.chunks, p.rows), dim3(kScanThreads), 0,
                     stream, static_cast<const T*>(logits), vocab, p.chunks, p.chunk_len, width,
                     part_max, part_sum, part_val, part_idx, err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const SelectLayout L = select_layout(depth_n, width, budget, WMAX);
  hipLaunchKernelGGL((tree_select<WMAX>), dim3(batch), dim3(kSelectThreads), L.bytes, stream,
                     part_max, part_sum, part_val, part_idx, p.chunks, depth_n, width, budget, L,
                     root_token, parent, token, depth, score, n_nodes, err);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_w(const void* logits, int batch, int depth_n, int vocab, int width,
                             int budget, const ScanPlan& p, const ScanWorkspace& w,
                             unsigned char* ws, const int32_t* root_token, int32_t* parent,
                             int32_t* token, int32_t* depth, double* score, int32_t* n_nodes,
                             int32_t* err, hipStream_t stream) {
#define JT_BUILD_CASE(WM)                                                                     \
  case WM:                                                                                   \
    return launch_build<T, WM>(logits, batch, depth_n, vocab, width, budget, p, w, ws,       \
                               root_token, parent, token, depth, score, n_nodes, err, stream);
  switch (p.wmax) {
    JT_BUILD_CASE(1)
    JT_BUILD_CASE(2)
    JT_BUILD_CASE(4)
    JT_BUILD_CASE(8)
    JT_BUILD_CASE(16)
  }
#undef JT_BUILD_CASE
  return hipErrorInvalidValue;
}

hipError_t build_tree_launch(const void* logits, jt_dtype dt, int batch, int depth_n, int vocab,
                             int width, int budget, const int32_t* root_token, int32_t* parent,
                             int32_t* token, int32_t* depth, double* score, int32_t* n_nodes,
                             int32_t* err, void* workspace, hipStream_t stream) {
  const ScanPlan p = scan_plan(batch, depth_n, vocab, width);
  const ScanWorkspace w = scan_workspace(p, width);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  if (dt == JT_F32)
    return dispatch_w<float>(logits, batch, depth_n, vocab, width, budget, p, w, ws, root_token,
                             parent, token, depth, score, n_nodes, err, stream);
  return dispatch_w<uint16_t>(logits, batch, depth_n, vocab, width, budget, p, w, ws, root_token,
                              parent, token, depth, score, n_nodes, err, stream);
}

}  // namespace jt
