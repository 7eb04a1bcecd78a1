// jt_accept_stochastic: lossless verification of the tree at temperature
// T > 0.  Single-token rule (SD overview, chooseai.io/news/6515, section on
// what speculative decoding is; AdaptiveSpec page, kongchang.com, section on
// the strict token-matching rule): accept a drafted token x with probability
// min(1, p(x)/q(x)); on rejection draw from norm(max(0, p - q)).
//
// Tree walk (one workgroup of 1024 threads per sequence): at the current
// node u, p = softmax(target row u / T); its children (node-index order = their
// candidate rank) are tried in turn; an accepted child becomes the current
// node; when none is accepted the bonus token is the inverse-CDF draw of
// u_sample over the current residual.  What q is depends on the proposal:
//
// * Top-W siblings (JT_DRAFT_TOPW; the trees jt_build_tree makes: JetSpec news
//   piece, tree-construction paragraph; explainer section 五).  The siblings
//   are chosen, so each one's proposal is the point mass on its token: x is
//   accepted iff u_accept < p_k(x), and a rejection removes x from p and
//   renormalises.  With et = exp((x - max) / T) of the target row (sum zt)
//   and R the rejected mass, p_k(x) = et[x] / (zt - R); a rejected token's
//   et entry is set to zero, so the bonus draw and a repeated token see it
//   removed.  No pass over the vocabulary follows a rejection.
// * Children drawn i.i.d. from q = softmax(draft row depth / T)
//   (JT_DRAFT_SAMPLED).  Child v (token x) is accepted iff
//   u_accept[v] * q(x) < p(x); a rejection replaces p by norm(max(0, p - q)).
//   With q fixed inside one node's child list, k rejections leave p_k
//   proportional to max(0, p - s_k q), s_0 = 0,
//   s_{k+1} = s_k + sum_y max(0, p - s_k q).  The kernel keeps that in
//   unnormalised form: with ed the exponentials of the draft row (sum zd) and
//   c = s zt / zd, the residual weights are max(0, et - c ed), their sum U,
//   and a rejection sets c += U / zd.  The accept test reads
//     u_accept * ed[x] / zd < max(0, et[x] - c ed[x]) / U,
//   the same inequality as u q(x) < p_k(x) up to rounding.  Every pass after
//   the row statistics is one fused multiply-add per entry.
// All probability arithmetic is fp64 (exp from the device math library).
//
// Every walk starts at the root (and, with sampled children, the depth-1
// draft row), so the statistics of those rows are computed beforehand across
// the whole GPU (chunk maxima, then the exponentials, per-chunk fp64 sums and
// counts of positive weights); the walk adds the chunk sums in chunk order and
// computes deeper rows itself.
#include "jt_device.h"
#include "jt_host.h"

namespace jt {

constexpr int kStThreads = 1024;
constexpr int kStWaves = kStThreads / kWave;
// Passes over the vocabulary load kStUnroll entries per thread before using
// them: one workgroup streams a whole row, so its loads in flight set the pace.
constexpr int kStUnroll = 8;
constexpr int kBonusBlocks = 4;  // blocks per wave segment of the bonus draw
constexpr int kPreThreads = 256;
constexpr int kPreChunk = kPreThreads * 16;  // entries of one pre-pass workgroup

// Workspace: et and ed (2 * vocab doubles per sequence), then per sequence
// and pre-pass row (0: the root's target row, 1: the depth-1 draft row) the
// chunk sums (double), maxima (float), bad flags (int) and counts of positive
// exponentials (int).
struct StWorkspace {
  size_t off_sum, off_max, off_bad, off_pos, bytes;
  int nch;
};

static __host__ __device__ StWorkspace st_workspace(int batch, int vocab) {
  StWorkspace w{};
  w.nch = (vocab + kPreChunk - 1) / kPreChunk;
  const size_t cells = static_cast<size_t>(batch) * 2 * w.nch;
  w.off_sum = (static_cast<size_t>(batch) * 2 * vocab * sizeof(double) + 255) / 256 * 256;
  w.off_max = w.off_sum + cells * sizeof(double);
  w.off_bad = w.off_max + cells * sizeof(float);
  w.off_pos = w.off_bad + cells * sizeof(int);
  w.bytes = w.off_pos + cells * sizeof(int);
  return w;
}

template <typename T>
__device__ __forceinline__ const T* pre_row(const T* target, const T* draft, int seq, int r,
                                            int max_nodes, int depth_n, int vocab) {
  return r == 0 ? target + static_cast<size_t>(seq) * max_nodes * vocab
                : draft + static_cast<size_t>(seq) * depth_n * vocab;
}

// Pre-pass 1: maximum and NaN / +inf flag of each chunk of the two rows.
template <typename T>
__global__ __launch_bounds__(kPreThreads) void stoch_pre_max(
    const T* __restrict__ target, const T* __restrict__ draft, int max_nodes, int vocab,
    int depth_n, int nch, int nrows, float* __restrict__ cmax, int* __restrict__ cbad) {
  __shared__ float rm[kPreThreads / kWave];
  __shared__ int rb[kPreThreads / kWave];
  // workgroup = (chunk, row, sequence), chunk fastest; nrows = 1 (root target
  // row only) or 2 (and the depth-1 draft row)
  const int c = blockIdx.x % nch, r = (blockIdx.x / nch) % nrows,
            seq = blockIdx.x / nch / nrows;
  const T* row = pre_row(target, draft, seq, r, max_nodes, depth_n, vocab);
  float m = -INFINITY;
  int b = 0;
  float x[kPreChunk / kPreThreads];
#pragma unroll
  for (int k = 0; k < kPreChunk / kPreThreads; ++k) {
    const int i = c * kPreChunk + k * kPreThreads + threadIdx.x;
    x[k] = i < vocab ? load_as_f32(row, i) : -INFINITY;
  }
#pragma unroll
  for (int k = 0; k < kPreChunk / kPreThreads; ++k) {
    if (x[k] != x[k] || x[k] == INFINITY) b = 1;
    m = fmaxf(m, x[k]);
  }
  for (int o = 32; o > 0; o >>= 1) {
    m = fmaxf(m, __shfl_xor(m, o, kWave));
    b |= __shfl_xor(b, o, kWave);
  }
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  if (lane == 0) { rm[wv] = m; rb[wv] = b; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kPreThreads / kWave; ++k) { m = fmaxf(m, rm[k]); b |= rb[k]; }
    const size_t cell = (static_cast<size_t>(seq) * 2 + r) * nch + c;
    cmax[cell] = m;
    cbad[cell] = b;
  }
}

// Pre-pass 2: row maximum from the chunk maxima, then exp((x - max) / T) into
// et (r = 0) or ed (r = 1), the chunk's fp64 sum (fixed summation order) and
// its count of positive exponentials.
template <typename T>
__global__ __launch_bounds__(kPreThreads) void stoch_pre_exp(
    const T* __restrict__ target, const T* __restrict__ draft, int max_nodes, int vocab,
    int depth_n, int nch, int nrows, double tinv, const float* __restrict__ cmax,
    const int* __restrict__ cbad, double* __restrict__ csum, int* __restrict__ cpos,
    double* __restrict__ ecache) {
  __shared__ double rs[kPreThreads / kWave];
  __shared__ int rp[kPreThreads / kWave];
  const int c = blockIdx.x % nch, r = (blockIdx.x / nch) % nrows,
            seq = blockIdx.x / nch / nrows;
  const size_t cell0 = (static_cast<size_t>(seq) * 2 + r) * nch;
  float m = -INFINITY;
  int b = 0;
  for (int k = 0; k < nch; ++k) { m = fmaxf(m, cmax[cell0 + k]); b |= cbad[cell0 + k]; }
  double z = 0.0;
  int pos = 0;
  if (!b && m != -INFINITY) {
    const T* row = pre_row(target, draft, seq, r, max_nodes, depth_n, vocab);
    double* e_out = ecache + (static_cast<size_t>(seq) * 2 + r) * vocab;
    float x[kPreChunk / kPreThreads];
#pragma unroll
    for (int k = 0; k < kPreChunk / kPreThreads; ++k) {
      const int i = c * kPreChunk + k * kPreThreads + threadIdx.x;
      x[k] = i < vocab ? load_as_f32(row, i) : m;
    }
#pragma unroll
    for (int k = 0; k < kPreChunk / kPreThreads; ++k) {
      const int i = c * kPreChunk + k * kPreThreads + threadIdx.x;
      if (i < vocab) {
        const double e = exp((static_cast<double>(x[k]) - static_cast<double>(m)) * tinv);
        e_out[i] = e;
        z += e;
        pos += e > 0.0;
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    z += __shfl_xor(z, o, kWave);
    pos += __shfl_xor(pos, o, kWave);
  }
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  if (lane == 0) { rs[wv] = z; rp[wv] = pos; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kPreThreads / kWave; ++k) { z += rs[k]; pos += rp[k]; }
    csum[cell0 + c] = z;
    cpos[cell0 + c] = pos;
  }
}

template <typename T>
struct RowView {
  const T* row;
  __device__ __forceinline__ float at(int i) const { return load_as_f32(row, i); }
  // entries 4j .. 4j + 3 in one load (the row must be 4-entry aligned)
  __device__ __forceinline__ void at4(int j, float* x) const;
};
template <>
__device__ __forceinline__ void RowView<float>::at4(int j, float* x) const {
  const float4 v = reinterpret_cast<const float4*>(row)[j];
  x[0] = v.x;
  x[1] = v.y;
  x[2] = v.z;
  x[3] = v.w;
}
template <>
__device__ __forceinline__ void RowView<uint16_t>::at4(int j, float* x) const {
  const uint2 v = reinterpret_cast<const uint2*>(row)[j];
  x[0] = bf16_bits_to_f32(static_cast<uint16_t>(v.x & 0xFFFFu));
  x[1] = bf16_bits_to_f32(static_cast<uint16_t>(v.x >> 16));
  x[2] = bf16_bits_to_f32(static_cast<uint16_t>(v.y & 0xFFFFu));
  x[3] = bf16_bits_to_f32(static_cast<uint16_t>(v.y >> 16));
}

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

__device__ __forceinline__ int block_add(int v, int* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  int t = 0;
  for (int k = 0; k < kStWaves; ++k) t += red[k];
  return t;
}

// Row statistics: max (exact) and Z = sum exp((x - max) / T) in fp64; every
// exp((x - max) / T) is also stored in e_out[i] for the later passes, and
// *pos_out counts the positive ones.  Sets *bad for NaN / +inf entries or a
// row without a finite entry.
template <typename T>
__device__ void row_stats(RowView<T> r, int vocab, double tinv, float* m_out, double* z_out,
                          int* pos_out, bool* bad, double* __restrict__ e_out, float* redf,
                          double* redd, int* redi) {
  float m = -INFINITY;
  int b = 0;
  // 4-entry loads when the row allows them (one load request per 4 entries:
  // a single workgroup streams the row, so its request rate sets the pace)
  const bool vec = (vocab & 3) == 0 && (reinterpret_cast<uintptr_t>(r.row) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(e_out) & 15) == 0;
  if (vec) {
    const int v4 = vocab / 4;
    for (int j0 = threadIdx.x; j0 < v4; j0 += kStThreads * 2) {
      float x[2][4];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int j = j0 + k * kStThreads;
        if (j < v4) r.at4(j, x[k]);
        else x[k][0] = x[k][1] = x[k][2] = x[k][3] = -INFINITY;
      }
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (x[k][e] != x[k][e] || x[k][e] == INFINITY) b = 1;
          m = fmaxf(m, x[k][e]);
        }
    }
  } else {
    for (int i0 = threadIdx.x; i0 < vocab; i0 += kStThreads * kStUnroll) {
      float x[kStUnroll];
#pragma unroll
      for (int k = 0; k < kStUnroll; ++k) {
        const int i = i0 + k * kStThreads;
        x[k] = i < vocab ? r.at(i) : -INFINITY;
      }
#pragma unroll
      for (int k = 0; k < kStUnroll; ++k) {
        if (x[k] != x[k] || x[k] == INFINITY) b = 1;
        m = fmaxf(m, x[k]);
      }
    }
  }
  m = block_max(m, redf);
  b = block_or(b, redi);
  double z = 0.0;
  int pos = 0;
  if (!b && m != -INFINITY && vec) {
    const int v4 = vocab / 4;
    double2* e2 = reinterpret_cast<double2*>(e_out);
    for (int j0 = threadIdx.x; j0 < v4; j0 += kStThreads * 2) {
      float x[2][4];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int j = j0 + k * kStThreads;
        if (j < v4) r.at4(j, x[k]);
        else x[k][0] = x[k][1] = x[k][2] = x[k][3] = m;
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int j = j0 + k * kStThreads;
        if (j < v4) {
          double e[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            e[q] = exp((static_cast<double>(x[k][q]) - static_cast<double>(m)) * tinv);
            z += e[q];
            pos += e[q] > 0.0;
          }
          e2[2 * j] = make_double2(e[0], e[1]);
          e2[2 * j + 1] = make_double2(e[2], e[3]);
        }
      }
    }
  } else if (!b && m != -INFINITY)
    for (int i0 = threadIdx.x; i0 < vocab; i0 += kStThreads * kStUnroll) {
      float x[kStUnroll];
#pragma unroll
      for (int k = 0; k < kStUnroll; ++k) {
        const int i = i0 + k * kStThreads;
        x[k] = i < vocab ? r.at(i) : m;
      }
#pragma unroll
      for (int k = 0; k < kStUnroll; ++k) {
        const int i = i0 + k * kStThreads;
        if (i < vocab) {
          const double e = exp((static_cast<double>(x[k]) - static_cast<double>(m)) * tinv);
          e_out[i] = e;
          z += e;
          pos += e > 0.0;
        }
      }
    }
  z = block_sum(z, redd);  // its barriers also publish e_out to the workgroup
  *pos_out = block_add(pos, redi);
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
    int32_t* __restrict__ bonus_token, int32_t* err, double* __restrict__ ecache,
    const double* __restrict__ pre_sum, const float* __restrict__ pre_max,
    const int* __restrict__ pre_bad, const int* __restrict__ pre_pos, int nch, int sampled) {
  __shared__ int par[1024];
  __shared__ float redf[kStWaves];
  __shared__ double redd[kStWaves];
  __shared__ int redi[kStWaves];
  __shared__ double bsum[kStWaves * kBonusBlocks], bpre[kStWaves * kBonusBlocks];
  __shared__ int owner_s;
  __shared__ int path[64];
  __shared__ int pick;
  __shared__ double thr_s;
  const int seq = blockIdx.x, tid = threadIdx.x;
  const int lane = tid % kWave, wv = tid / kWave;
  const int n = n_nodes[seq];
  int32_t* nodes_out = accept_nodes + static_cast<size_t>(seq) * depth_n;
  // exp((x - max) / T) of the current target row and of the children's draft row
  double* et = ecache + static_cast<size_t>(seq) * 2 * vocab;
  double* ed = et + vocab;
  // the cached rows can be read as 16-byte entry pairs
  const bool pairs = (vocab & 1) == 0 && (reinterpret_cast<uintptr_t>(et) & 15) == 0;
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
  b = block_or(b, redi);
  if (b) { fail(b); return; }

  const double tinv = 1.0 / static_cast<double>(temperature);
  // statistics of pre-pass row r (0: root target row, 1: depth-1 draft row),
  // whose exponentials are already in et / ed; chunk sums added in order
  auto pre_stats = [&](int r, float* m_out, double* z_out, int* pos_out, bool* bad) {
    const size_t cell0 = (static_cast<size_t>(seq) * 2 + r) * nch;
    float m = -INFINITY;
    int bb = 0, pos = 0;
    double z = 0.0;
    for (int k = 0; k < nch; ++k) {
      m = fmaxf(m, pre_max[cell0 + k]);
      bb |= pre_bad[cell0 + k];
      z += pre_sum[cell0 + k];
      pos += pre_pos[cell0 + k];
    }
    *m_out = m;
    *z_out = z;
    *pos_out = pos;
    *bad = bb || m == -INFINITY;
  };
  int u = 0, L = 0;
  // current distribution: weights max(0, et - c ed) over the current node's
  // target row (ed: the children's draft row), total U; c = 0 is plain p
  float mt = 0.0f, md = 0.0f;
  double zt = 1.0, zd = 1.0, c = 0.0, U = 1.0;
  int npos = 0, npos_d = 0;
  auto node_stats = [&](bool* bad) {
    if (u == 0)
      pre_stats(0, &mt, &zt, &npos, bad);
    else
      row_stats(RowView<T>{target + (base + u) * vocab}, vocab, tinv, &mt, &zt, &npos, bad, et,
                redf, redd, redi);
  };
  while (!sampled) {
    // top-W siblings: point-mass proposals.  zt - R is the mass left after
    // the rejected tokens (whose et entries are then zero).
    bool bad = false;
    node_stats(&bad);
    if (bad) { fail(JT_DERR_BAD_LOGIT); return; }
    double R = 0.0;
    int npos_rej = 0;
    int next = -1;
    for (int v = u + 1; v < n; ++v) {
      if (par[v] != u) continue;  // uniform: par is in LDS, v is uniform
      const int x = token[base + v];
      const double ex = et[x];
      // the mass left still holds x itself (guards the rounding of zt - R)
      if (static_cast<double>(u_accept[base + v]) < ex / fmax(zt - R, ex)) {
        next = v;
        break;
      }
      if (ex > 0.0) {
        // removing the last positive weight would leave no mass: keep p
        if (npos_rej + 1 == npos) break;
        ++npos_rej;
        R += ex;
        __syncthreads();  // every thread has read et[x]
        if (tid == 0) et[x] = 0.0;
        __syncthreads();  // the removal is visible to later reads
      }
    }
    if (next < 0) break;
    if (tid == 0) path[L] = next;
    ++L;
    u = next;
    __syncthreads();  // every thread is done with et before the next row overwrites it
  }
  const T* draft_seq = sampled ? draft + static_cast<size_t>(seq) * depth_n * vocab : nullptr;
  while (sampled) {
    bool bad = false;
    node_stats(&bad);
    if (bad) { fail(JT_DERR_BAD_LOGIT); return; }
    c = 0.0;
    U = zt;
    bool have_q = false;  // ed holds the children's draft row (all at depth(u) + 1)
    int next = -1;
    for (int v = u + 1; v < n; ++v) {
      if (par[v] != u) continue;  // uniform: par is in LDS, v is uniform
      if (!have_q) {
        const int d = depth[base + v];
        if (d == 1)
          pre_stats(1, &md, &zd, &npos_d, &bad);
        else
          row_stats(RowView<T>{draft_seq + static_cast<size_t>(d - 1) * vocab}, vocab, tinv, &md,
                    &zd, &npos_d, &bad, ed, redf, redd, redi);
        if (bad) { fail(JT_DERR_BAD_LOGIT); return; }
        have_q = true;
      }
      const int x = token[base + v];
      const double qx = ed[x] / zd;
      const double pcur = fmax(0.0, et[x] - c * ed[x]) / U;
      if (static_cast<double>(u_accept[base + v]) * qx < pcur) {
        next = v;
        break;
      }
      // rejection: c' = c + U / zd, U' = sum_y max(0, et - c' ed)
      const double c_new = c + U / zd;
      double part = 0.0;
      if (pairs) {
        // 16-byte loads of entry pairs, 4 pairs per thread in flight
        const double2* et2 = reinterpret_cast<const double2*>(et);
        const double2* ed2 = reinterpret_cast<const double2*>(ed);
        const int v2 = vocab / 2;
        for (int i0 = tid; i0 < v2; i0 += kStThreads * (kStUnroll / 2)) {
          double2 a[kStUnroll / 2], q[kStUnroll / 2];
#pragma unroll
          for (int k = 0; k < kStUnroll / 2; ++k) {
            const int i = i0 + k * kStThreads;
            a[k] = i < v2 ? et2[i] : make_double2(0.0, 0.0);
            q[k] = i < v2 ? ed2[i] : make_double2(0.0, 0.0);
          }
#pragma unroll
          for (int k = 0; k < kStUnroll / 2; ++k) {
            part += fmax(0.0, a[k].x - c_new * q[k].x);
            part += fmax(0.0, a[k].y - c_new * q[k].y);
          }
        }
      } else {
        for (int i0 = tid; i0 < vocab; i0 += kStThreads * kStUnroll) {
          double a[kStUnroll], q[kStUnroll];
#pragma unroll
          for (int k = 0; k < kStUnroll; ++k) {
            const int i = i0 + k * kStThreads;
            a[k] = i < vocab ? et[i] : 0.0;
            q[k] = i < vocab ? ed[i] : 0.0;
          }
#pragma unroll
          for (int k = 0; k < kStUnroll; ++k) part += fmax(0.0, a[k] - c_new * q[k]);
        }
      }
      const double un = block_sum(part, redd);
      if (un == 0.0) break;  // no mass left: keep the previous distribution
      c = c_new;
      U = un;
    }
    if (next < 0) break;
    if (tid == 0) path[L] = next;
    ++L;
    u = next;
    __syncthreads();  // every thread is done with et before the next row overwrites it
  }
  // ---- bonus: inverse-CDF draw over the residual weights of the current node
  // (c == 0: the weights are et itself, with top-W rejections already zeroed).
  // Wave w owns a contiguous segment of the vocabulary, cut into kBonusBlocks
  // blocks (lanes read them coalesced).  One exclusive prefix over the block
  // sums in (wave, block) order finds the block whose interval holds
  // u * total (the intervals tile [0, total) exactly: they come from the same
  // fp64 additions), and that block's wave scans it 64 entries at a time.
  auto weight = [&](int i) -> double { return c == 0.0 ? et[i] : fmax(0.0, et[i] - c * ed[i]); };
  const int seg = (vocab + kStWaves * kWave - 1) / (kStWaves * kWave) * kWave;
  const int s0 = min(vocab, wv * seg), s1 = min(vocab, s0 + seg);
  const int blen = ((seg + kBonusBlocks - 1) / kBonusBlocks + kWave - 1) / kWave * kWave;
  double own[kBonusBlocks];
#pragma unroll
  for (int bb = 0; bb < kBonusBlocks; ++bb) {
    const int b0 = min(s1, s0 + bb * blen), b1 = min(s1, b0 + blen);
    double acc = 0.0;
    if (pairs) {
      // 16-byte loads of entry pairs (blocks start and, with an even
      // vocabulary, end at even entries)
      const double2* et2 = reinterpret_cast<const double2*>(et);
      const double2* ed2 = reinterpret_cast<const double2*>(ed);
      for (int i0 = b0 / 2 + lane; i0 < b1 / 2; i0 += kWave * (kStUnroll / 2)) {
        double2 a[kStUnroll / 2], q[kStUnroll / 2];
#pragma unroll
        for (int k = 0; k < kStUnroll / 2; ++k) {
          const int i = i0 + k * kWave;
          a[k] = i < b1 / 2 ? et2[i] : make_double2(0.0, 0.0);
          q[k] = (c != 0.0 && i < b1 / 2) ? ed2[i] : make_double2(0.0, 0.0);
        }
#pragma unroll
        for (int k = 0; k < kStUnroll / 2; ++k) {
          acc += c == 0.0 ? a[k].x : fmax(0.0, a[k].x - c * q[k].x);
          acc += c == 0.0 ? a[k].y : fmax(0.0, a[k].y - c * q[k].y);
        }
      }
    } else {
      for (int i0 = b0 + lane; i0 < b1; i0 += kWave * kStUnroll) {
        double w[kStUnroll];
#pragma unroll
        for (int k = 0; k < kStUnroll; ++k) {
          const int i = i0 + k * kWave;
          w[k] = i < b1 ? weight(i) : 0.0;
        }
#pragma unroll
        for (int k = 0; k < kStUnroll; ++k) acc += w[k];
      }
    }
    own[bb] = acc;
  }
#pragma unroll
  for (int bb = 0; bb < kBonusBlocks; ++bb) {
    double v = own[bb];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    if (lane == 0) bsum[wv * kBonusBlocks + bb] = v;
  }
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
    for (int k = 0; k < kStWaves * kBonusBlocks; ++k) {
      bpre[k] = tot;  // exclusive prefix
      tot += bsum[k];
    }
    const double thr = static_cast<double>(u_sample[seq]) * tot;
    int o = -1;
    for (int k = 0; k < kStWaves * kBonusBlocks && o < 0; ++k)
      if (bpre[k] <= thr && bpre[k] + bsum[k] > thr) o = k;
    thr_s = thr;
    owner_s = o;
    pick = -1;
  }
  __syncthreads();
  const double thr = thr_s;
  const int owner = owner_s;
  if (owner >= 0 && wv == owner / kBonusBlocks) {
    const int bb = owner % kBonusBlocks;
    const int b0 = min(s1, s0 + bb * blen), b1 = min(s1, b0 + blen);
    double carry = bpre[owner];
    int y = -1, last_pos = -1;
    // 64-entry chunks in order, kStUnroll chunks loaded at a time
    for (int c0 = b0; c0 < b1 && y < 0; c0 += kWave * kStUnroll) {
      double wk[kStUnroll];
#pragma unroll
      for (int k = 0; k < kStUnroll; ++k) {
        const int i = c0 + k * kWave + lane;
        wk[k] = i < b1 ? weight(i) : 0.0;
      }
#pragma unroll
      for (int k = 0; k < kStUnroll; ++k) {
        const int r0 = c0 + k * kWave;
        if (y >= 0 || r0 >= b1) break;  // wave-uniform
        const double w = wk[k];
        double incl = w;  // inclusive prefix over the 64 lanes
        for (int o = 1; o < kWave; o <<= 1) {
          const double up = __shfl_up(incl, o, kWave);
          if (lane >= o) incl += up;
        }
        const unsigned long long hit = __ballot(carry + incl > thr);
        const unsigned long long pos = __ballot(w > 0.0);
        if (pos) last_pos = r0 + 63 - __clzll(pos);
        if (hit) y = r0 + __ffsll(static_cast<long long>(hit)) - 1;
        carry += __shfl(incl, kWave - 1, kWave);
      }
    }
    if (lane == 0) pick = y >= 0 ? y : last_pos;  // re-summation rounding: last positive weight
  }
  __syncthreads();
  if (tid == 0) {
    bonus_token[seq] = pick;
    accept_len[seq] = L;
    for (int k = 0; k < depth_n; ++k) nodes_out[k] = (k < L) ? path[k] : -1;
  }
}

size_t accept_stochastic_workspace_bytes(int batch, int vocab) {
  return st_workspace(batch, vocab).bytes;
}

hipError_t accept_stochastic_launch(const void* target, const void* draft, jt_dtype dt,
                                    int batch, int max_nodes, int vocab, int depth_n,
                                    const int32_t* parent, const int32_t* token,
                                    const int32_t* depth, const int32_t* n_nodes,
                                    float temperature, const float* u_accept,
                                    const float* u_sample, int sampled, int32_t* accept_len,
                                    int32_t* accept_nodes, int32_t* bonus_token, int32_t* err,
                                    void* workspace, hipStream_t stream) {
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  double* ecache = reinterpret_cast<double*>(ws);
  const StWorkspace L = st_workspace(batch, vocab);
  double* csum = reinterpret_cast<double*>(ws + L.off_sum);
  float* cmax = reinterpret_cast<float*>(ws + L.off_max);
  int* cbad = reinterpret_cast<int*>(ws + L.off_bad);
  int* cpos = reinterpret_cast<int*>(ws + L.off_pos);
  const double tinv = 1.0 / static_cast<double>(temperature);
  // rows computed up front: the root's target row, plus the depth-1 draft row
  // when children are sampled from the draft
  const int nrows = sampled ? 2 : 1;
  const dim3 pre_grid(static_cast<unsigned>(L.nch) * static_cast<unsigned>(nrows) *
                      static_cast<unsigned>(batch));
#define JT_ST_LAUNCH(TT)                                                                        \
  do {                                                                                          \
    const TT* tg = static_cast<const TT*>(target);                                              \
    const TT* dr = static_cast<const TT*>(draft);                                               \
    hipLaunchKernelGGL(stoch_pre_max<TT>, pre_grid, dim3(kPreThreads), 0, stream, tg, dr,       \
                       max_nodes, vocab, depth_n, L.nch, nrows, cmax, cbad);                    \
    hipLaunchKernelGGL(stoch_pre_exp<TT>, pre_grid, dim3(kPreThreads), 0, stream, tg, dr,       \
                       max_nodes, vocab, depth_n, L.nch, nrows, tinv, cmax, cbad, csum, cpos,   \
                       ecache);                                                                 \
    hipLaunchKernelGGL(accept_stochastic_kernel<TT>, dim3(batch), dim3(kStThreads), 0, stream,  \
                       tg, dr, max_nodes, vocab, depth_n, parent, token, depth, n_nodes,        \
                       temperature, u_accept, u_sample, accept_len, accept_nodes, bonus_token,  \
                       err, ecache, csum, cmax, cbad, cpos, L.nch, sampled);                    \
  } while (0)
  if (dt == JT_F32)
    JT_ST_LAUNCH(float);
  else
    JT_ST_LAUNCH(uint16_t);
#undef JT_ST_LAUNCH
  return hipGetLastError();
}

}  // namespace jt
