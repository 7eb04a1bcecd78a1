// jt_accept_stochastic: lossless verification of the tree at temperature
// T > 0.  Single-token rule (SD overview, chooseai.io/news/6515, section on
// what speculative decoding is; AdaptiveSpec page, kongchang.com, section on
// the strict token-matching rule): accept a drafted token x with probability
// min(1, p(x)/q(x)); on rejection draw from norm(max(0, p - q)).
//
// Tree walk (one workgroup of 1024 threads per sequence): at the current
// node u, p = softmax(target row u / T); its children (node-index order = their
// candidate rank) are tried in turn with q = softmax(draft row depth / T) of
// their depth: child v (token x) is accepted iff u_accept[v] * q(x) < p(x);
// a rejection replaces p by norm(max(0, p - q)).  With q fixed inside one
// node's child list, after k rejections p_k = max(0, p - s_k q) / N_k with
// s_0 = 0, N_0 = 1, s_k = s_{k-1} + N_{k-1} and
// N_k = sum_y max(0, p(y) - s_k q(y)), so each rejection costs one fp64 pass
// over the vocabulary.  When no child is accepted the bonus token is the
// inverse-CDF draw of u_sample from the current p.  All probability
// arithmetic is fp64 (exp from the device math library).
#include "jt_device.h"
#include "jt_host.h"

namespace jt {

constexpr int kStThreads = 1024;
constexpr int kStWaves = kStThreads / kWave;

template <typename T>
struct RowView {
  const T* row;
  __device__ __forceinline__ float at(int i) const { return load_as_f32(row, i); }
};

// fp64 block sum (every thread gets the result); red: kStWaves doubles
__device__ __forceinline__ double block_sum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  double t = 0.0;
  for (int k = 0; k < kStWaves; ++k) t += red[k];
  return t;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int k = 0; k < kStWaves; ++k) t = fmaxf(t, red[k]);
  return t;
}

__device__ __forceinline__ int block_or(int v, int* red) {
  for (int o = 32; o > 0; o >>= 1) v |= __shfl_xor(v, o, kWave);
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  int t = 0;
  for (int k = 0; k < kStWaves; ++k) t |= red[k];
  return t;
}

// Row statistics: max (exact) and Z = sum exp((x - max) / T) in fp64.  Sets
// *bad for NaN / +inf entries or a row without a finite entry.
template <typename T>
__device__ void row_stats(RowView<T> r, int vocab, double tinv, float* m_out, double* z_out,
                          bool* bad, float* redf, double* redd, int* redi) {
  float m = -INFINITY;
  int b = 0;
  for (int i = threadIdx.x; i < vocab; i += kStThreads) {
    const float x = r.at(i);
    if (x != x || x == INFINITY) b = 1;
    m = fmaxf(m, x);
  }
  m = block_max(m, redf);
  b = block_or(b, redi);
  double z = 0.0;
  if (!b && m != -INFINITY)
    for (int i = threadIdx.x; i < vocab; i += kStThreads)
      z += exp((static_cast<double>(r.at(i)) - static_cast<double>(m)) * tinv);
  z = block_sum(z, redd);
  *m_out = m;
  *z_out = z;
  *bad = b || m == -INFINITY;
}

template <typename T>
__global__ __launch_bounds__(kStThreads) void accept_stochastic_kernel(
    const T* __restrict__ target, const T* __restrict__ draft, int max_nodes, int vocab,
    int depth_n, const int32_t* __restrict__ parent, const int32_t* __restrict__ token,
    const int32_t* __restrict__ depth, const int32_t* __restrict__ n_nodes, float temperature,
    const float* __restrict__ u_accept, const float* __restrict__ u_sample,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ accept_nodes,
    int32_t* __restrict__ bonus_token, int32_t* err) {
  __shared__ int par[1024];
  __shared__ float dmax[64];
  __shared__ double dz[64];
  __shared__ int dstate[64];  // 0 unknown, 1 valid, 2 bad
  __shared__ float redf[kStWaves];
  __shared__ double redd[kStWaves];
  __shared__ int redi[kStWaves];
  __shared__ double chunk_pre[kStThreads];
  __shared__ int path[64];
  const int seq = blockIdx.x, tid = threadIdx.x;
  const int n = n_nodes[seq];
  int32_t* nodes_out = accept_nodes + static_cast<size_t>(seq) * depth_n;
  auto fail = [&](int bits) {
    if (tid == 0) {
      report(err, bits);
      accept_len[seq] = 0;
      bonus_token[seq] = -1;
    }
    for (int k = tid; k < depth_n; k += kStThreads) nodes_out[k] = -1;
  };
  if (n < 1 || n > max_nodes) { fail(JT_DERR_BAD_NNODES); return; }
  const size_t base = static_cast<size_t>(seq) * max_nodes;
  // ---- validate the tree, tokens and uniforms
  int b = 0;
  for (int v = tid; v < n; v += kStThreads) {
    const int p = parent[base + v];
    par[v] = p;
    const int d = depth[base + v];
    if (v == 0) {
      if (p != -1 || d != 0) b |= JT_DERR_BAD_PARENT;
    } else {
      if (p < 0 || p >= v) b |= JT_DERR_BAD_PARENT;
      else if (d != depth[base + p] + 1 || d > depth_n) b |= JT_DERR_BAD_DEPTH;
      const int t = token[base + v];
      if (t < 0 || t >= vocab) b |= JT_DERR_BAD_TOKEN;
      const float ua = u_accept[base + v];
      if (!(ua >= 0.0f && ua < 1.0f)) b |= JT_DERR_BAD_UNIFORM;
    }
  }
  if (tid == 0) {
    const float us = u_sample[seq];
    if (!(us >= 0.0f && us < 1.0f)) b |= JT_DERR_BAD_UNIFORM;
  }
  for (int k = tid; k < 64; k += kStThreads) dstate[k] = 0;
  b = block_or(b, redi);
  if (b) { fail(b); return; }

  const double tinv = 1.0 / static_cast<double>(temperature);
  const T* draft_seq = draft + static_cast<size_t>(seq) * depth_n * vocab;
  int u = 0, L = 0;
  // current distribution: p_cur(y) = max(0, p(y) - s q(y)) / N over the
  // current node's target row (q of the children's depth; s = 0: plain p)
  float mt = 0.0f, md = 0.0f;
  double zt = 1.0, zd = 1.0, s = 0.0, N = 1.0;
  int qdepth = 0;  // draft row of q (1-based depth), 0: no q term
  while (true) {
    bool bad = false;
    RowView<T> tr{target + (base + u) * vocab};
    row_stats(tr, vocab, tinv, &mt, &zt, &bad, redf, redd, redi);
    if (bad) { fail(JT_DERR_BAD_LOGIT); return; }
    s = 0.0;
    N = 1.0;
    qdepth = 0;
    int next = -1;
    for (int v = u + 1; v < n; ++v) {
      if (par[v] != u) continue;  // uniform: par is in LDS, v is uniform
      const int d = depth[base + v];
      if (dstate[d - 1] == 0) {
        RowView<T> dr{draft_seq + static_cast<size_t>(d - 1) * vocab};
        float m;
        double z;
        row_stats(dr, vocab, tinv, &m, &z, &bad, redf, redd, redi);
        __syncthreads();
        if (tid == 0) {
          dmax[d - 1] = m;
          dz[d - 1] = z;
          dstate[d - 1] = bad ? 2 : 1;
        }
        __syncthreads();
      }
      if (dstate[d - 1] == 2) { fail(JT_DERR_BAD_LOGIT); return; }
      md = dmax[d - 1];
      zd = dz[d - 1];
      qdepth = d;
      const T* drow = draft_seq + static_cast<size_t>(d - 1) * vocab;
      const int x = token[base + v];
      const double px = exp((static_cast<double>(load_as_f32(tr.row, x)) - mt) * tinv) / zt;
      const double qx = exp((static_cast<double>(load_as_f32(drow, x)) - md) * tinv) / zd;
      const double pcur = fmax(0.0, px - s * qx) / N;
      if (static_cast<double>(u_accept[base + v]) * qx < pcur) {
        next = v;
        break;
      }
      // rejection: N_new = sum_y max(0, p(y) - (s + N) q(y))
      const double s_new = s + N;
      double part = 0.0;
      for (int i = tid; i < vocab; i += kStThreads) {
        const double py = exp((static_cast<double>(tr.at(i)) - mt) * tinv) / zt;
        const double qy = exp((static_cast<double>(load_as_f32(drow, i)) - md) * tinv) / zd;
        part += fmax(0.0, py - s_new * qy);
      }
      const double nn = block_sum(part, redd);
      if (nn == 0.0) break;  // no mass left: keep the previous distribution
      s = s_new;
      N = nn;
    }
    if (next < 0) break;
    if (tid == 0) path[L] = next;
    ++L;
    u = next;
  }
  // ---- bonus: inverse-CDF draw from p_cur over the current node's row
  const T* trow = target + (base + u) * vocab;
  const T* drow = qdepth > 0 ? draft_seq + static_cast<size_t>(qdepth - 1) * vocab : nullptr;
  const int chunk = (vocab + kStThreads - 1) / kStThreads;
  const int lo = min(vocab, tid * chunk), hi = min(vocab, lo + chunk);
  auto weight = [&](int i) -> double {
    const double py = exp((static_cast<double>(load_as_f32(trow, i)) - mt) * tinv) / zt;
    if (s == 0.0) return py;
    const double qy = exp((static_cast<double>(load_as_f32(drow, i)) - md) * tinv) / zd;
    return fmax(0.0, py - s * qy);
  };
  double own = 0.0;
  for (int i = lo; i < hi; ++i) own += weight(i);
  chunk_pre[tid] = own;
  __syncthreads();
  __shared__ int pick;
  __shared__ double thr_s;
  if (tid == 0) {
    double tot = 0.0;
    for (int k = 0; k < kStThreads; ++k) {
      const double c = chunk_pre[k];
      chunk_pre[k] = tot;  // exclusive prefix
      tot += c;
    }
    thr_s = static_cast<double>(u_sample[seq]) * tot;
    pick = -1;
  }
  __syncthreads();
  const double thr = thr_s;
  // The chunk intervals [pre_k, pre_k + own_k) tile [0, tot) exactly (the
  // same fp64 additions as the prefix), so exactly one thread owns thr.
  if (lo < hi && chunk_pre[tid] <= thr && chunk_pre[tid] + own > thr) {
    double run = chunk_pre[tid];
    int y = -1, last_pos = -1;
    for (int i = lo; i < hi; ++i) {
      const double wi = weight(i);
      if (wi > 0.0) last_pos = i;
      run += wi;
      if (run > thr) { y = i; break; }
    }
    pick = y >= 0 ? y : last_pos;  // re-summation rounding: last positive weight of the chunk
  }
  __syncthreads();
  if (tid == 0) {
    bonus_token[seq] = pick;
    accept_len[seq] = L;
    for (int k = 0; k < depth_n; ++k) nodes_out[k] = (k < L) ? path[k] : -1;
  }
}

hipError_t accept_stochastic_launch(const void* target, const void* draft, jt_dtype dt,
                                    int batch, int max_nodes, int vocab, int depth_n,
                                    const int32_t* parent, const int32_t* token,
                                    const int32_t* depth, const int32_t* n_nodes,
                                    float temperature, const float* u_accept,
                                    const float* u_sample, int32_t* accept_len,
                                    int32_t* accept_nodes, int32_t* bonus_token, int32_t* err,
                                    hipStream_t stream) {
  if (dt == JT_F32)
    hipLaunchKernelGGL(accept_stochastic_kernel<float>, dim3(batch), dim3(kStThreads), 0, stream,
                       static_cast<const float*>(target), static_cast<const float*>(draft),
                       max_nodes, vocab, depth_n, parent, token, depth, n_nodes, temperature,
                       u_accept, u_sample, accept_len, accept_nodes, bonus_token, err);
  else
    hipLaunchKernelGGL(accept_stochastic_kernel<uint16_t>, dim3(batch), dim3(kStThreads), 0,
                       stream, static_cast<const uint16_t*>(target),
                       static_cast<const uint16_t*>(draft), max_nodes, vocab, depth_n, parent,
                       token, depth, n_nodes, temperature, u_accept, u_sample, accept_len,
                       accept_nodes, bonus_token, err);
  return hipGetLastError();
}

}  // namespace jt
