// jt_tree_attention: paged tree-causal attention of every tree node in one
// pass (JetSpec explainer, techwalker.com "加速AI思考…", section 七: paged
// tree attention with the tree mask staged on chip and the tree tail masked,
// never a dense mask; section 三: all candidate paths verified in one target
// forward; JetSpec news piece, mlqm.cn/news/158889: the tree-causal mask).
//
// bf16 path (tree_attn_mfma): one workgroup = 4 waves x 32 query rows for one
// (sequence, KV head, row tile, key split).  Query rows are (node, head of the
// GQA group) pairs, node-major, so every K/V tile staged in LDS is reused by
// all the group's query heads and tree nodes.  Per 64-key tile:
//   * K and V of 4 pages are gathered from the paged pool with 16-byte loads
//     (register double buffering), K stored [key][dim] with an XOR swizzle, V
//     stored transposed [dim][key] with an XOR swizzle;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys as M, queries as N, so
//     each lane owns one query column and the softmax reductions stay
//     in-lane plus one cross-half exchange);
//   * online softmax in base 2 with a lazy rescale (the running max is only
//     moved when a tile exceeds it by more than 2^8);
//   * O^T += V^T P^T on the same MFMA, P taken straight from the S^T
//     registers (the key order inside each 16-key step is permuted to match
//     the accumulator layout, and V^T is read in the same order).
// Only tiles that reach the tree tail apply the mask: the lane's node reads a
// 64-bit window of its ancestor bitmask.  Tail tiles past the tile's last node
// are skipped (a node never sees a later node).  Long key ranges are split
// across workgroups; a combine kernel merges the partial (o, lse) pairs.
//
// f32 path (tree_attn_f32): one wave per (sequence, node, query head), keys
// across lanes; exact fp32 arithmetic, used for fp32 inputs.
#include "jt_device.h"
#include "jt_host.h"

#include <algorithm>
#include <cmath>

namespace jt {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kKT = 64;            // keys per tile
constexpr int kWavesM = 4;         // waves per workgroup
constexpr int kRowsWave = 32;      // query rows per wave
constexpr int kRowsWG = kWavesM * kRowsWave;
constexpr int kAttnThreads = kWavesM * kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* n_nodes;
  const int32_t* prefix_len;
  const int32_t* page_table;
  const uint32_t* anc;
  uint16_t* out;
  float* lse;
  float* part_o;    // [batch, hkv, splits, rows_pad, D] (splits > 1)
  float* part_lse;  // [batch, hkv, splits, rows_pad]
  int32_t* err;
  int max_nodes, hq, hkv, group, max_pages, num_pages, splits, row_tiles, rows_pad, nwords;
  float scale_log2;  // scale * log2(e)
};

__device__ __forceinline__ int vt_swz(int d) { return ((d >> 3) + 2 * (d & 7)) & 15; }

// Validates one sequence; returns false (and reports) when it must be skipped.
__device__ __forceinline__ bool seq_ok(int n, int P, int max_nodes, int max_pages, int32_t* err,
                                       bool reporter) {
  if (n < 1 || n > max_nodes) {
    if (reporter) report(err, JT_DERR_BAD_NNODES);
    return false;
  }
  if (P < 0 || static_cast<long long>(P) + n > static_cast<long long>(max_pages) * kPage) {
    if (reporter) report(err, JT_DERR_BAD_PREFIX);
    return false;
  }
  return true;
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void tree_attn_mfma(AttnArgs a) {
  constexpr int CPK = D / 8;                 // 16-byte chunks per key row
  constexpr int KLD = kKT * CPK / kAttnThreads;  // K chunk loads per thread
  constexpr int VQ = kKT / 4;                // key quads per tile
  constexpr int VTHREADS = VQ * CPK;         // threads that stage V
  constexpr int DB = D / 32;                 // 32-row blocks of O^T
  constexpr int KS = D / 16;                 // MFMA k-steps of QK^T

  __shared__ __align__(16) uint16_t k_lds[2][kKT * D];
  __shared__ __align__(16) uint16_t vt_lds[2][D * kKT];

  const int s = blockIdx.z, g = blockIdx.y;
  const int rt = blockIdx.x / a.splits, sp = blockIdx.x % a.splits;
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int h = lane >> 5, col = lane & 31;

  const int n = a.n_nodes[s];
  const int P = a.prefix_len[s];
  if (!seq_ok(n, P, a.max_nodes, a.max_pages, a.err, blockIdx.x == 0 && g == 0 && tid == 0)) return;
  const int rows = n * a.group;
  const int rowbase = rt * kRowsWG;
  if (rowbase >= rows) return;
  const int node_hi = min(n - 1, (rowbase + kRowsWG - 1) / a.group);
  const int key_end = P + node_hi + 1;                 // causal skip of later nodes
  const int ntiles = (key_end + kKT - 1) / kKT;
  const int tb = static_cast<int>(static_cast<long long>(ntiles) * sp / a.splits);
  const int te = static_cast<int>(static_cast<long long>(ntiles) * (sp + 1) / a.splits);

  // ---- this lane's query row
  const int r = rowbase + w * kRowsWave + col;
  const bool row_ok = r < rows;
  const int node = row_ok ? r / a.group : 0;
  const int hq = g * a.group + (row_ok ? r % a.group : 0);
  bf16x8 qreg[KS];
  {
    const uint16_t* qp = a.q + ((static_cast<size_t>(s) * a.max_nodes + node) * a.hq + hq) * D;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row_ok) u = *reinterpret_cast<const uint4*>(qp + 16 * kk + 8 * h);
      qreg[kk] = __builtin_bit_cast(bf16x8, u);
    }
  }
  const uint32_t* anc_row = a.anc + (static_cast<size_t>(s) * a.max_nodes + node) * a.nwords;

  const int32_t* ptab = a.page_table + static_cast<size_t>(s) * a.max_pages;
  const size_t head_stride = static_cast<size_t>(kPage) * D;           // one page of one head
  const size_t page_stride = static_cast<size_t>(a.hkv) * head_stride;

  // ---- global -> register staging of one tile
  uint4 kst[KLD];
  uint4 vst[4];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int e = tid + i * kAttnThreads;
      const int key = e / CPK, c = e % CPK;
      const int t = t0 + key;
      uint4 u = make_uint4(0, 0, 0, 0);
      if (t < P + n) {
        const int page = ptab[t / kPage];
        if (page >= 0 && page < a.num_pages) {
          u = *reinterpret_cast<const uint4*>(a.k_pool + page * page_stride + g * head_stride +
                                               (t % kPage) * D + c * 8);
        } else {
          report(a.err, JT_DERR_BAD_PAGE);
        }
      }
      kst[i] = u;
    }
    if (tid < VTHREADS) {
      const int c = tid % CPK, kq = tid / CPK;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = t0 + 4 * kq + j;
        uint4 u = make_uint4(0, 0, 0, 0);
        if (t < P + n) {
          const int page = ptab[t / kPage];
          if (page >= 0 && page < a.num_pages)
            u = *reinterpret_cast<const uint4*>(a.v_pool + page * page_stride + g * head_stride +
                                                 (t % kPage) * D + c * 8);
        }
        vst[j] = u;
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int e = tid + i * kAttnThreads;
      const int key = e / CPK, c = e % CPK;
      *reinterpret_cast<uint4*>(&k_lds[buf][key * D + ((c ^ (key & 7)) * 8)]) = kst[i];
    }
    if (tid < VTHREADS) {
      const int c = tid % CPK, kq = tid / CPK;
      const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vst[0]);
      const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vst[1]);
      const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&vst[2]);
      const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&vst[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * c + e;
        const int sh = (e & 1) ? 16 : 0;
        const uint32_t x0 = (v0[e >> 1] >> sh) & 0xFFFFu, x1 = (v1[e >> 1] >> sh) & 0xFFFFu;
        const uint32_t x2 = (v2[e >> 1] >> sh) & 0xFFFFu, x3 = (v3[e >> 1] >> sh) & 0xFFFFu;
        uint2 pk;
        pk.x = x0 | (x1 << 16);
        pk.y = x2 | (x3 << 16);
        const int pq = kq ^ vt_swz(d);
        *reinterpret_cast<uint2*>(&vt_lds[buf][d * kKT + pq * 4]) = pk;
      }
    }
  };

  f32x16 o_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o_acc[db][v] = 0.0f;
  float m_run = -INFINITY;  // running max in scaled (log2) units
  float l_run = 0.0f;       // this lane's half of the normaliser

  if (tb < te) {
    fetch(tb * kKT);
    stash(0);
  }
  __syncthreads();
  for (int it = tb; it < te; ++it) {
    const int buf = (it - tb) & 1;
    const int t0 = it * kKT;
    if (it + 1 < te) fetch(t0 + kKT);

    // ---- S^T = K Q^T for 2 blocks of 32 keys
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.0f;
      const int key = kb * 32 + col;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int c = 2 * kk + h;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(&k_lds[buf][key * D + ((c ^ (key & 7)) * 8)]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[kk], sacc[kb], 0, 0, 0);
      }
    }

    // ---- mask (tiles that reach the tree tail)
    if (t0 + kKT > P) {
      const int jb = t0 - P;  // tail index of the tile's first key (may be < 0)
      uint64_t win = 0;
      {
        const int w0 = (jb >= 0) ? (jb >> 5) : -((-jb + 31) >> 5);
        const int sh = jb - 32 * w0;  // 0..31
        uint32_t wd[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const int wi = w0 + k;
          wd[k] = (row_ok && wi >= 0 && wi < a.nwords) ? anc_row[wi] : 0u;
        }
        const uint64_t lo = (static_cast<uint64_t>(wd[1]) << 32) | wd[0];
        win = (lo >> sh) | (sh ? (static_cast<uint64_t>(wd[2]) << (64 - sh)) : 0ull);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int o = kb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
          const int t = t0 + o;
          const bool vis = (t < P) || ((win >> o) & 1ull);
          if (!vis) sacc[kb][v] = -INFINITY;
        }
    }

    // ---- online softmax (base 2, lazy rescale)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mx_s = mx * a.scale_log2;
    const bool need = (m_run == -INFINITY) ? (mx_s != -INFINITY) : (mx_s > m_run + kRescaleThreshold);
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? mx_s : m_run;
      const float alpha = need ? ((m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new)) : 1.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o_acc[db][v] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float base = (m_run == -INFINITY) ? 0.0f : m_run;
    bf16x8 pf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = exp2f(fmaf(sacc[kb][v], a.scale_log2, -base));
        l_run += p;
        pf[kb * 2 + (v >> 3)][v & 7] = static_cast<__bf16>(p);
      }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d = db * 32 + col;
      const int sw = vt_swz(d);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kb = ks >> 1, j = ks & 1;
        const int qa = 8 * kb + 4 * j + h;
        const int qb = qa + 2;
        const uint2 lo = *reinterpret_cast<const uint2*>(&vt_lds[buf][d * kKT + (qa ^ sw) * 4]);
        const uint2 hi = *reinterpret_cast<const uint2*>(&vt_lds[buf][d * kKT + (qb ^ sw) * 4]);
        const uint4 u = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), pf[ks],
                                                            o_acc[db], 0, 0, 0);
      }
    }

    if (it + 1 < te) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
  const float lse_v = (l_tot > 0.0f) ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  if (!row_ok) return;
  if (a.splits == 1) {
    uint16_t* op = a.out + ((static_cast<size_t>(s) * a.max_nodes + node) * a.hq + hq) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d0 = db * 32 + 8 * grp + 4 * h;
        uint2 pk;
        const __bf16 b0 = static_cast<__bf16>(o_acc[db][4 * grp + 0] * inv);
        const __bf16 b1 = static_cast<__bf16>(o_acc[db][4 * grp + 1] * inv);
        const __bf16 b2 = static_cast<__bf16>(o_acc[db][4 * grp + 2] * inv);
        const __bf16 b3 = static_cast<__bf16>(o_acc[db][4 * grp + 3] * inv);
        pk.x = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b0)) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b1)) << 16);
        pk.y = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b2)) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b3)) << 16);
        *reinterpret_cast<uint2*>(op + d0) = pk;
      }
    if (a.lse && h == 0)
      a.lse[(static_cast<size_t>(s) * a.max_nodes + node) * a.hq + hq] = lse_v;
  } else {
    const size_t prow = ((static_cast<size_t>(s) * a.hkv + g) * a.splits + sp) * a.rows_pad + r;
    float* op = a.part_o + prow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d0 = db * 32 + 8 * grp + 4 * h;
        *reinterpret_cast<float4*>(op + d0) =
            make_float4(o_acc[db][4 * grp] * inv, o_acc[db][4 * grp + 1] * inv,
                        o_acc[db][4 * grp + 2] * inv, o_acc[db][4 * grp + 3] * inv);
      }
    if (h == 0) a.part_lse[prow] = lse_v;
  }
}

// Merges the per-split partials of every (sequence, KV head, row).
template <int D>
__global__ __launch_bounds__(256) void tree_attn_combine(AttnArgs a) {
  constexpr int TPR = 64;  // threads per row
  constexpr int PER = D / TPR;
  const int s = blockIdx.z, g = blockIdx.y;
  const int r = blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  const int n = a.n_nodes[s];
  const int P = a.prefix_len[s];
  if (!seq_ok(n, P, a.max_nodes, a.max_pages, a.err, false)) return;
  if (r >= n * a.group) return;
  const int node = r / a.group, hq = g * a.group + r % a.group;
  const size_t base = (static_cast<size_t>(s) * a.hkv + g) * a.splits;
  float M = -INFINITY;
  for (int sp = 0; sp < a.splits; ++sp) M = fmaxf(M, a.part_lse[(base + sp) * a.rows_pad + r]);
  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
  float wsum = 0.0f;
  for (int sp = 0; sp < a.splits; ++sp) {
    const size_t prow = (base + sp) * a.rows_pad + r;
    const float ls = a.part_lse[prow];
    if (ls == -INFINITY) continue;
    const float wgt = expf(ls - M);
    wsum += wgt;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] += wgt * a.part_o[prow * D + t + k * TPR];
  }
  const float inv = 1.0f / wsum;
  uint16_t* op = a.out + ((static_cast<size_t>(s) * a.max_nodes + node) * a.hq + hq) * D;
#pragma unroll
  for (int k = 0; k < PER; ++k)
    op[t + k * TPR] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[k] * inv));
  if (a.lse && t == 0)
    a.lse[(static_cast<size_t>(s) * a.max_nodes + node) * a.hq + hq] = M + logf(wsum);
}

// fp32 inputs: one wave per (sequence, node, query head); 64 keys per step
// across the lanes, exact fp32 online softmax.
template <int D>
__global__ __launch_bounds__(kWave) void tree_attn_f32(
    const float* __restrict__ q, const float* __restrict__ k_pool, const float* __restrict__ v_pool,
    const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ prefix_len,
    const int32_t* __restrict__ page_table, const uint32_t* __restrict__ anc, float scale,
    float* __restrict__ out, float* __restrict__ lse, int32_t* err, int max_nodes, int hq,
    int hkv, int max_pages, int num_pages, int nwords) {
  constexpr int PER = D / kWave;
  __shared__ float qs[D];
  const int node = blockIdx.x, h = blockIdx.y, s = blockIdx.z, lane = threadIdx.x;
  const int n = n_nodes[s];
  const int P = prefix_len[s];
  if (!seq_ok(n, P, max_nodes, max_pages, err, node == 0 && h == 0 && lane == 0)) return;
  if (node >= n) return;
  const int g = h / (hq / hkv);
  const float* qp = q + ((static_cast<size_t>(s) * max_nodes + node) * hq + h) * D;
  for (int d = lane; d < D; d += kWave) qs[d] = qp[d];
  __syncthreads();
  const uint32_t* arow = anc + (static_cast<size_t>(s) * max_nodes + node) * nwords;
  const int32_t* ptab = page_table + static_cast<size_t>(s) * max_pages;
  const size_t hs = static_cast<size_t>(kPage) * D, ps = hkv * hs;
  float m = -INFINITY, l = 0.0f, o[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) o[k] = 0.0f;
  const int key_end = P + node + 1;
  for (int t0 = 0; t0 < key_end; t0 += kWave) {
    const int t = t0 + lane;
    bool vis = t < key_end && (t < P || ((arow[(t - P) >> 5] >> ((t - P) & 31)) & 1u));
    const float* krow = nullptr;
    if (vis) {
      const int page = ptab[t / kPage];
      if (page < 0 || page >= num_pages) { report(err, JT_DERR_BAD_PAGE); vis = false; }
      else krow = k_pool + page * ps + g * hs + (t % kPage) * D;
    }
    float sc = -INFINITY;
    if (vis) {
      float dot = 0.0f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], krow[d], dot);
      sc = dot * scale;
    }
    float mx = sc;
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) continue;
    const float alpha = (m == -INFINITY) ? 0.0f : expf(m - m_new);
    const float p = vis ? expf(sc - m_new) : 0.0f;
    float ps_sum = p;
    for (int off = 32; off > 0; off >>= 1) ps_sum += __shfl_xor(ps_sum, off, kWave);
    l = l * alpha + ps_sum;
#pragma unroll
    for (int k = 0; k < PER; ++k) o[k] *= alpha;
    m = m_new;
    for (int j = 0; j < kWave; ++j) {
      const float pj = __shfl(p, j, kWave);
      if (pj == 0.0f) continue;  // uniform across the wave
      const int tj = t0 + j;
      const int page = ptab[tj / kPage];
      const float* vrow = v_pool + page * ps + g * hs + (tj % kPage) * D;
#pragma unroll
      for (int k = 0; k < PER; ++k) o[k] = fmaf(pj, vrow[lane + k * kWave], o[k]);
    }
  }
  float* op = out + ((static_cast<size_t>(s) * max_nodes + node) * hq + h) * D;
#pragma unroll
  for (int k = 0; k < PER; ++k) op[lane + k * kWave] = o[k] / l;
  if (lse && lane == 0) lse[(static_cast<size_t>(s) * max_nodes + node) * hq + h] = m + logf(l);
}

// ------------------------------------------------------------------ host side

struct AttnPlan {
  int row_tiles, rows_pad, splits;
  size_t off_lse, bytes;
};

static AttnPlan attn_plan(const AttnShape& s) {
  AttnPlan p{};
  const int group = s.hq / s.hkv;
  p.row_tiles = (s.max_nodes * group + kRowsWG - 1) / kRowsWG;
  p.rows_pad = p.row_tiles * kRowsWG;
  const long long base = static_cast<long long>(p.row_tiles) * s.hkv * s.batch;
  const int tiles = (s.max_pages * s.page_size + kKT - 1) / kKT;
  const long long want = (512 + base - 1) / std::max<long long>(1, base);
  p.splits = static_cast<int>(std::max<long long>(1, std::min<long long>(want, std::min(tiles, 32))));
  if (s.dt == JT_F32) p.splits = 1;
  if (p.splits > 1) {
    const size_t rows = static_cast<size_t>(s.batch) * s.hkv * p.splits * p.rows_pad;
    p.off_lse = (rows * s.head_dim * sizeof(float) + 255) / 256 * 256;
    p.bytes = p.off_lse + (rows * sizeof(float) + 255) / 256 * 256;
  }
  return p;
}

size_t tree_attention_workspace_bytes(const AttnShape& s) {
  if (s.batch <= 0) return 0;
  return attn_plan(s).bytes;
}

template <int D>
static hipError_t launch_mfma(const AttnShape& sh, const AttnPlan& p, AttnArgs& a,
                              hipStream_t stream) {
  hipLaunchKernelGGL(tree_attn_mfma<D>, dim3(p.row_tiles * p.splits, sh.hkv, sh.batch),
                     dim3(kAttnThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  hipLaunchKernelGGL(tree_attn_combine<D>, dim3(p.rows_pad / 4, sh.hkv, sh.batch), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t tree_attention_launch(const AttnShape& sh, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* n_nodes,
                                 const int32_t* prefix_len, const int32_t* page_table,
                                 const uint32_t* anc_mask, float scale, void* out, float* lse,
                                 int32_t* err, void* workspace, hipStream_t stream) {
  const int nwords = (sh.max_nodes + 31) / 32;
  if (sh.dt == JT_F32) {
#define JT_F32_LAUNCH(DD)                                                                     \
  hipLaunchKernelGGL(tree_attn_f32<DD>, dim3(sh.max_nodes, sh.hq, sh.batch), dim3(kWave), 0, \
                     stream, static_cast<const float*>(q), static_cast<const float*>(k_pool), \
                     static_cast<const float*>(v_pool), n_nodes, prefix_len, page_table,      \
                     anc_mask, scale, static_cast<float*>(out), lse, err, sh.max_nodes, sh.hq, \
                     sh.hkv, sh.max_pages, sh.num_pages, nwords)
    if (sh.head_dim == 64) JT_F32_LAUNCH(64); else JT_F32_LAUNCH(128);
#undef JT_F32_LAUNCH
    return hipGetLastError();
  }
  const AttnPlan p = attn_plan(sh);
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.v_pool = static_cast<const uint16_t*>(v_pool);
  a.n_nodes = n_nodes;
  a.prefix_len = prefix_len;
  a.page_table = page_table;
  a.anc = anc_mask;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.part_o = p.splits > 1 ? static_cast<float*>(workspace) : nullptr;
  a.part_lse = p.splits > 1
                   ? reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + p.off_lse)
                   : nullptr;
  a.err = err;
  a.max_nodes = sh.max_nodes;
  a.hq = sh.hq;
  a.hkv = sh.hkv;
  a.group = sh.hq / sh.hkv;
  a.max_pages = sh.max_pages;
  a.num_pages = sh.num_pages;
  a.splits = p.splits;
  a.row_tiles = p.row_tiles;
  a.rows_pad = p.rows_pad;
  a.nwords = nwords;
  a.scale_log2 = scale * kLog2e;
  if (sh.head_dim == 64) return launch_mfma<64>(sh, p, a, stream);
  return launch_mfma<128>(sh, p, a, stream);
}

}  // namespace jt
