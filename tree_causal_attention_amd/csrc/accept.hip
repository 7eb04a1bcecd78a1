// jt_accept: greedy acceptance of the longest consistent path.
//
// JetSpec news piece (mlqm.cn/news/158889): the target verifies the whole tree
// in one pass and keeps the longest prefix consistent with the SD acceptance
// rule; JetSpec explainer section 三 (the longest accepted prefix along each
// candidate path); SD overview (chooseai.io/news/6515), section on when
// "lossless" fails: at temperature 0 a draft token is accepted only when it
// equals the target's choice.
//
// row_argmax: one workgroup per (vocab chunk, tree row, sequence) streams the
//   target logits of rows < n_nodes once with 16-byte non-temporal loads
//   (HBM-bound; the rows are not reused) and keeps the best (value, lowest id).
// accept_walk: one workgroup per sequence, one thread per node: merges the
//   chunk winners, marks accepted nodes level by level (parent < child, so a
//   level only reads the previous one) and picks the deepest accepted node.
//   The same walk runs the margin rule of jt_accept_margin (AdaptiveSpec page,
//   kongchang.com, section on the per-step margin rule): a drafted token is
//   kept when its target probability over the top-1's reaches a threshold.
#include "jt_device.h"
#include "jt_host.h"

#include <algorithm>
#include <mutex>

namespace jt {

constexpr int kArgmaxThreads = 256;       // threads of an argmax workgroup on small grids
constexpr int kArgmaxThreadsLarge = 512;  // ... and on grids of at least kLargeArgmaxGrid
// With a grid of many workgroups the wider shape streams the chunks faster
// (each thread's chain of dependent load rounds is half as long); small grids
// keep 256 threads.
constexpr long long kLargeArgmaxGrid = 1024;
// 16-byte vectors for the streaming loads (read once: non-temporal)
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
constexpr int kWalkThreads = 1024;

template <typename T, int VEC, int NT>
__global__ __launch_bounds__(NT) void row_argmax(
    const T* __restrict__ logits, const int32_t* __restrict__ n_nodes, int max_nodes, int vocab,
    int chunks, int chunk_len, float* __restrict__ part_val, int* __restrict__ part_idx,
    int32_t* err) {
  const int c = blockIdx.x, row = blockIdx.y, seq = blockIdx.z;
  const int n = n_nodes[seq];
  if (n < 1 || n > max_nodes || row >= n) return;
  const T* x = logits + (static_cast<size_t>(seq) * max_nodes + row) * vocab;
  const int begin = c * chunk_len;
  const int end = min(vocab, begin + chunk_len);
  float bv = -INFINITY;
  int bi = INT32_MAX;
  bool bad = false;
  if (VEC > 1) {
    // begin and end are multiples of VEC here (host guarantees vocab % VEC == 0
    // and chunk_len % VEC == 0), and rows start VEC-aligned.  UNR loads per
    // thread are issued before any of them is consumed.
    constexpr int UNR = 4;
    for (int i0 = begin + threadIdx.x * VEC; i0 < end; i0 += NT * VEC * UNR) {
      float v[UNR][VEC];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int i = i0 + u * NT * VEC;
        if (i < end) {
          if constexpr (sizeof(T) == 4) {
            const f32x4v f = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(x + i));
            v[u][0] = f.x; v[u][1] = f.y; v[u][2] = f.z; v[u][3] = f.w;
          } else {
            const u32x4v q = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(x + i));
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              v[u][2 * k] = __uint_as_float(w[k] << 16);
              v[u][2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
            }
          }
        } else {
#pragma unroll
          for (int k = 0; k < VEC; ++k) v[u][k] = -INFINITY;
        }
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int i = i0 + u * NT * VEC;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
          const float y = v[u][k];
          if (y != y) { bad = true; continue; }
          if (i + k < end && better(y, i + k, bv, bi)) { bv = y; bi = i + k; }
        }
      }
    }
  } else {
    for (int i = begin + threadIdx.x; i < end; i += NT) {
      const float v = load_as_f32(x, i);
      if (v != v) { bad = true; continue; }
      if (better(v, i, bv, bi)) { bv = v; bi = i; }
    }
  }
  if (bad) report(err, JT_DERR_BAD_LOGIT);
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = shfl_xor(bv, o);
    const int oi = shfl_xor(bi, o);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  __shared__ float sv[NT / kWave];
  __shared__ int si[NT / kWave];
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  if (lane == 0) { sv[wv] = bv; si[wv] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < NT / kWave; ++w)
      if (better(sv[w], si[w], bv, bi)) { bv = sv[w]; bi = si[w]; }
    const size_t o = (static_cast<size_t>(seq) * max_nodes + row) * chunks + c;
    part_val[o] = bv;
    part_idx[o] = bi;
  }
}

// mode 0 (greedy): node v is accepted iff its parent is and token[v] equals the
//   parent row's argmax.
// mode 1 (margin): node v is accepted iff its parent is and
//   (double)L[parent][token[v]] - (double)max L[parent] >= margin (fp64, exact
//   difference of the stored values); the logit is gathered from `logits`.
template <typename T>
__global__ __launch_bounds__(kWalkThreads) void accept_walk(
    const float* __restrict__ part_val, const int* __restrict__ part_idx, int chunks,
    int max_nodes, int depth_n, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ token, const int32_t* __restrict__ depth,
    const int32_t* __restrict__ n_nodes, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ accept_nodes, int32_t* __restrict__ bonus_token, int32_t* err,
    const T* __restrict__ logits, int vocab, int mode, double margin) {
  __shared__ int a[1024];
  __shared__ float mx[1024];
  __shared__ int par[1024];
  __shared__ int dep[1024];
  __shared__ unsigned char acc[1024];
  __shared__ int bad;
  __shared__ unsigned int best_key;
  const int seq = blockIdx.x, v = threadIdx.x;
  const size_t base = static_cast<size_t>(seq) * max_nodes;
  // Every slot's inputs are loaded while the node count is still in flight
  // (each array spans max_nodes per sequence; slots past the count hold stale
  // values that are never used).  The chunk winners are loaded kBatch at a
  // time, all loads before the first comparison.
  constexpr int kBatch = 8;
  float bv = -INFINITY;
  int bi = INT32_MAX, pv = -1, dv = 0, tv = 0;
  if (v < max_nodes) {
    pv = parent[base + v];
    dv = depth[base + v];
    tv = token[base + v];
    const size_t o = (base + v) * chunks;
    for (int c0 = 0; c0 < chunks; c0 += kBatch) {
      float cv[kBatch];
      int ci[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int c = min(c0 + k, chunks - 1);  // repeats of the last chunk change nothing
        cv[k] = part_val[o + c];
        ci[k] = part_idx[o + c];
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k)
        if (better(cv[k], ci[k], bv, bi)) { bv = cv[k]; bi = ci[k]; }
    }
  }
  const int n = n_nodes[seq];
  int32_t* nodes_out = accept_nodes + static_cast<size_t>(seq) * depth_n;
  if (n < 1 || n > max_nodes) {
    if (v == 0) {
      report(err, JT_DERR_BAD_NNODES);
      accept_len[seq] = 0;
      bonus_token[seq] = -1;
    }
    for (int k = v; k < depth_n; k += kWalkThreads) nodes_out[k] = -1;
    return;
  }
  if (v == 0) { bad = 0; best_key = 0u; }
  __syncthreads();
  if (v < n) {
    a[v] = bi;
    mx[v] = bv;
    par[v] = pv;
    dep[v] = dv;
    acc[v] = (v == 0) ? 1 : 0;
  }
  __syncthreads();
  if (v < n) {
    int b = 0;
    if (v == 0) {
      if (par[0] != -1 || dep[0] != 0) b = JT_DERR_BAD_PARENT;
    } else {
      const int p = par[v];
      if (p < 0 || p >= v) b = JT_DERR_BAD_PARENT;
      else if (dep[v] != dep[p] + 1 || dep[v] > depth_n) b = JT_DERR_BAD_DEPTH;
      else if (mode == 1 && (tv < 0 || tv >= vocab)) b = JT_DERR_BAD_TOKEN;
    }
    if (b) atomicOr(&bad, b);
  }
  __syncthreads();
  if (bad) {
    if (v == 0) {
      report(err, bad);
      accept_len[seq] = 0;
      bonus_token[seq] = -1;
    }
    for (int k = v; k < depth_n; k += kWalkThreads) nodes_out[k] = -1;
    return;
  }
  // this node's own test on its parent's row (one gathered logit in margin mode)
  bool pass = false;
  if (v < n && v > 0) {
    const int p = par[v];
    const int t = tv;
    if (mode == 0) {
      pass = t == a[p];
    } else {
      const double lt = static_cast<double>(load_as_f32(logits, (base + p) * vocab + t));
      pass = lt - static_cast<double>(mx[p]) >= margin;
    }
  }
  for (int lvl = 1; lvl <= depth_n; ++lvl) {
    if (v < n && dep[v] == lvl) acc[v] = (acc[par[v]] && pass) ? 1 : 0;
    __syncthreads();
  }
  if (v < n && acc[v])
    atomicMax(&best_key, (static_cast<unsigned int>(dep[v]) << 16) | (0xFFFFu - v));
  __syncthreads();
  if (v == 0) {
    const int end = static_cast<int>(0xFFFFu - (best_key & 0xFFFFu));
    const int L = dep[end];
    int u = end;
    for (int k = L - 1; k >= 0; --k) { nodes_out[k] = u; u = par[u]; }
    for (int k = L; k < depth_n; ++k) nodes_out[k] = -1;
    accept_len[seq] = L;
    bonus_token[seq] = a[end];
  }
}

// ------------------------------------------------------------------ host side

struct ArgmaxPlan {
  int chunks, chunk_len, vec;
};

static ArgmaxPlan argmax_plan(int batch, int max_nodes, int vocab, int vec_elems) {
  ArgmaxPlan p{};
  const long long rows = static_cast<long long>(batch) * max_nodes;
  const int by_rows = static_cast<int>(std::max<long long>(1, (2048 + rows - 1) / std::max<long long>(1, rows)));
  const int by_vocab = std::max(1, (vocab + 4095) / 4096);
  // at least 8 chunks per row: with one workgroup per row the last few rows
  // run alone after the rest and stream at one workgroup's memory parallelism
  p.chunks = std::min(64, std::min(std::max(by_rows, 8), by_vocab));
  p.vec = (vocab % vec_elems == 0) ? vec_elems : 1;
  int len = (vocab + p.chunks - 1) / p.chunks;
  len = (len + p.vec - 1) / p.vec * p.vec;
  p.chunk_len = len;
  p.chunks = (vocab + len - 1) / len;
  return p;
}

static void argmax_ws(int batch, int max_nodes, const ArgmaxPlan& p, size_t* off_idx,
                      size_t* bytes) {
  const size_t n = static_cast<size_t>(batch) * max_nodes * p.chunks;
  const size_t a = (n * sizeof(float) + 255) / 256 * 256;
  *off_idx = a;
  *bytes = a + (n * sizeof(int) + 255) / 256 * 256;
}

size_t accept_workspace_bytes(int batch, int max_nodes, int vocab) {
  if (batch <= 0) return 0;
  // the f32 plan has the most chunks of the two dtypes' plans
  const ArgmaxPlan p4 = argmax_plan(batch, max_nodes, vocab, 4);
  const ArgmaxPlan p8 = argmax_plan(batch, max_nodes, vocab, 8);
  size_t o, b4, b8;
  argmax_ws(batch, max_nodes, p4, &o, &b4);
  argmax_ws(batch, max_nodes, p8, &o, &b8);
  return std::max(b4, b8);
}

template <typename T, int VEC>
static void launch_argmax(const void* logits, int batch, int max_nodes, int vocab,
                          const ArgmaxPlan& p, const int32_t* n_nodes, float* pv, int* pi,
                          int32_t* err, hipStream_t stream) {
  const dim3 grid(p.chunks, max_nodes, batch);
  if (static_cast<long long>(p.chunks) * max_nodes * batch >= kLargeArgmaxGrid)
    hipLaunchKernelGGL((row_argmax<T, VEC, kArgmaxThreadsLarge>), grid, dim3(kArgmaxThreadsLarge),
                       0, stream, static_cast<const T*>(logits), n_nodes, max_nodes, vocab,
                       p.chunks, p.chunk_len, pv, pi, err);
  else
    hipLaunchKernelGGL((row_argmax<T, VEC, kArgmaxThreads>), grid, dim3(kArgmaxThreads), 0, stream,
                       static_cast<const T*>(logits), n_nodes, max_nodes, vocab, p.chunks,
                       p.chunk_len, pv, pi, err);
}

// Scratch of the no-allocation entry point: the argmax partials live in this
// array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in): the device address comes
// from hipGetSymbolAddress, looked up once per device with that device
// current, and is cached here.
static __device__ __align__(256) unsigned char scratch[kAcceptScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxScratchDevices] = {};
}  // namespace

hipError_t accept_scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

hipError_t accept_launch(const void* logits, jt_dtype dt, int batch, int max_nodes, int vocab,
                         int depth_n, const int32_t* parent, const int32_t* token,
                         const int32_t* depth, const int32_t* n_nodes, int32_t* accept_len,
                         int32_t* accept_nodes, int32_t* bonus_token, int32_t* err,
                         void* workspace, hipStream_t stream, int mode, double margin) {
  ArgmaxPlan p = argmax_plan(batch, max_nodes, vocab, dt == JT_F32 ? 4 : 8);
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0) p.vec = 1;  // rows not 16-byte aligned
  size_t off_idx, bytes;
  argmax_ws(batch, max_nodes, p, &off_idx, &bytes);
  float* pv = static_cast<float*>(workspace);
  int* pi = reinterpret_cast<int*>(static_cast<unsigned char*>(workspace) + off_idx);
  if (dt == JT_F32) {
    if (p.vec == 4) launch_argmax<float, 4>(logits, batch, max_nodes, vocab, p, n_nodes, pv, pi, err, stream);
    else launch_argmax<float, 1>(logits, batch, max_nodes, vocab, p, n_nodes, pv, pi, err, stream);
  } else {
    if (p.vec == 8) launch_argmax<uint16_t, 8>(logits, batch, max_nodes, vocab, p, n_nodes, pv, pi, err, stream);
    else launch_argmax<uint16_t, 1>(logits, batch, max_nodes, vocab, p, n_nodes, pv, pi, err, stream);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dt == JT_F32)
    hipLaunchKernelGGL(accept_walk<float>, dim3(batch), dim3(kWalkThreads), 0, stream, pv, pi,
                       p.chunks, max_nodes, depth_n, parent, token, depth, n_nodes, accept_len,
                       accept_nodes, bonus_token, err, static_cast<const float*>(logits), vocab,
                       mode, margin);
  else
    hipLaunchKernelGGL(accept_walk<uint16_t>, dim3(batch), dim3(kWalkThreads), 0, stream, pv,
                       pi, p.chunks, max_nodes, depth_n, parent, token, depth, n_nodes,
                       accept_len, accept_nodes, bonus_token, err,
                       static_cast<const uint16_t*>(logits), vocab, mode, margin);
  return hipGetLastError();
}

}  // namespace jt
