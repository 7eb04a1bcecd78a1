// draft_row_scan: the per-depth statistics of the tree build (jt_build_tree,
// jt_build_tree_variant): fp64 log-sum-exp and the top-W tokens of every
// draft row, and optionally the fp64 entropy partials.
//
// Method: JetSpec news piece (mlqm.cn/news/158889), tree-construction
// paragraph (top-W candidates per depth, scored by log-probability); JetSpec
// explainer (techwalker.com, "加速AI思考…"), section 五 (the entropy
// priority the variants rank by).
//
// One workgroup per (vocab chunk, depth row) reads its chunk once with 16-byte
// loads; the partials of a row are merged by the select kernels.
#include "jt_device.h"
#include "jt_host.h"

namespace jt {

constexpr int kScanThreads = 256;       // threads of a scan workgroup on large grids
constexpr int kScanThreadsSmall = 512;  // ... and on grids of at most kSmallScanGrid
// Chunks are 8K logits either way; grids this small (one or two sequences)
// finish sooner with the chunk spread over twice the threads (16 logits a
// thread), larger ones sooner with 256 threads of 32 logits.
constexpr int kSmallScanGrid = 512;

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

// e^y in fp64 for finite y <= 0, table-driven (Tang's method): y = k c + r
// with c = ln2 / 256, |r| <= c / 2, so e^y = 2^(k >> 8) * 2^((k & 255) / 256)
// * e^r; the table holds 2^(j / 256) and e^r is its degree-5 Taylor
// polynomial (truncation below 2^-64 relative).  c is split into a 32-bit
// head (k * c_hi is exact for |k| < 2^21, i.e. y > -5600) and a tail.
__device__ __forceinline__ double exp_nonpos(double y, const double* __restrict__ exp2_tbl) {
  constexpr double kInvC = 369.3299304675746;       // 256 / ln2
  constexpr double kCHi = 0.00270760617331689;      // ln2 / 256, leading 32 bits
  constexpr double kCLo = 7.453964567463233e-13;    // ln2 / 256 - kCHi
  const double kd = rint(y * kInvC);
  const double r = fma(-kd, kCLo, fma(-kd, kCHi, y));
  const int k = static_cast<int>(kd);
  double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(exp2_tbl[k & 255] * p, k >> 8);
}

// One workgroup per (vocab chunk, depth row); thread t holds EPT logits of
// the chunk in registers (16-byte loads, one pass over HBM).
//  * max and the fp64 sum of exp(x - max) come straight from the registers;
//  * top-W: each wave offers its ceil(WMAX/4) largest lane maxima (distinct
//    logits of the chunk); the W-th largest offer L is a lower bound of the
//    chunk's W-th largest logit, so only logits >= L are collected in LDS and
//    ranked; if more than kCandCap qualify (e.g. massive ties) every thread
//    builds its exact sorted top-W and W rounds of "best head" merge them.
// ENT: also the fp64 sum of exp(x - max) * (x - max) (the chunk's entropy
// partial; tree_select_seq merges it into the per-depth entropy).
template <typename T, int WMAX, int VEC, int EPT, bool ENT, int NT>
__global__ __launch_bounds__(NT) void draft_row_scan(
    const T* __restrict__ logits, int vocab, int chunks, int chunk_len, int width,
    float* __restrict__ part_max, double* __restrict__ part_sum, double* __restrict__ part_ent,
    float* __restrict__ part_val, int* __restrict__ part_idx, int32_t* err) {
  constexpr int NV = EPT / VEC;
  __shared__ float sm_m[NT / kWave];
  __shared__ double sm_s[NT / kWave];
  __shared__ double sm_t[NT / kWave];
  constexpr int PW = (WMAX + 3) / 4;  // threshold offers per wave
  __shared__ float sm_off[(NT / kWave) * PW];
  __shared__ float sm_cv[kCandCap];
  __shared__ int sm_ci[kCandCap];
  __shared__ int sm_n;
  __shared__ float sm_L;
  __shared__ float sm_v[NT / kWave];
  __shared__ int sm_i[NT / kWave];
  __shared__ double sm_exp2[256];  // 2^(j / 256)
  static_assert(NT >= 256, "one table entry a thread");

  const int row = blockIdx.y, c = blockIdx.x, t = threadIdx.x;
  if (t < 256) sm_exp2[t] = exp2(static_cast<double>(t) * (1.0 / 256.0));
  const int lane = t % kWave, wv = t / kWave;
  const int begin = c * chunk_len;
  const int end = min(vocab, begin + chunk_len);
  const T* x = logits + static_cast<size_t>(row) * vocab;

  float xv[EPT];
  bool bad = false;
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = begin + (j * NT + t) * VEC;
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
  {
    // the wave's PW largest lane maxima (ties to the lower lane), one per round
    bool taken = false;
    for (int r = 0; r < PW; ++r) {
      float bv = taken ? -INFINITY : m;
      int bl = taken ? kWave : lane;  // taken lanes lose every comparison
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = shfl_xor(bv, o);
        const int ol = shfl_xor(bl, o);
        if (ov > bv || (ov == bv && ol < bl)) { bv = ov; bl = ol; }
      }
      if (lane == bl) taken = true;
      if (lane == 0) sm_off[wv * PW + r] = bl < kWave ? bv : -INFINITY;
    }
  }
  __syncthreads();
  float M = sm_m[0];
  for (int w = 1; w < NT / kWave; ++w) M = fmaxf(M, sm_m[w]);

  // ---- fp64 sum of exp(x - M) over the registers
  double sacc = 0.0, tacc = 0.0;
  if (M != -INFINITY) {
    const double Md = static_cast<double>(M);
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      // x >= -1e30: dx is finite, and e^dx underflows to 0 well before the
      // table method's range ends; -inf entries are dropped below
      const double dx = fmax(static_cast<double>(fmaxf(xv[k], -1.0e30f)) - Md, -5000.0);
      double e;
      if constexpr (EPT <= 32) e = exp_nonpos(dx, sm_exp2);
      else e = exp(dx);  // long chunks (vocab > 2^19): the table code unrolled 128x compiles slowly
      const bool fin = xv[k] != -INFINITY;
      sacc += fin ? e : 0.0;
      if constexpr (ENT) tacc += fin ? e * dx : 0.0;
    }
  }
  for (int o = 32; o > 0; o >>= 1) sacc += shfl_xor_f64(sacc, o);
  if (lane == 0) sm_s[wv] = sacc;
  if constexpr (ENT) {
    for (int o = 32; o > 0; o >>= 1) tacc += shfl_xor_f64(tacc, o);
    if (lane == 0) sm_t[wv] = tacc;
  }

  // ---- threshold: the W-th largest of the 4 * PW offers (ties by position)
  if (t < (NT / kWave) * PW) {
    const float v = sm_off[t];
    int rank = 0;
    for (int u = 0; u < (NT / kWave) * PW; ++u) {
      const float ou = sm_off[u];
      rank += (ou > v || (ou == v && u < t)) ? 1 : 0;
    }
    if (rank == width - 1) sm_L = v;
  }
  __syncthreads();
  if (t == 0) {
    double S = 0.0;
    for (int w = 0; w < NT / kWave; ++w) S += sm_s[w];
    part_max[row * chunks + c] = M;
    part_sum[row * chunks + c] = S;
    if constexpr (ENT) {
      double Tt = 0.0;
      for (int w = 0; w < NT / kWave; ++w) Tt += sm_t[w];
      part_ent[row * chunks + c] = Tt;
    }
  }
  const float L = sm_L;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int i = begin + (j * NT + t) * VEC;
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
    for (int q = t; q < nc; q += NT) {
      const float vq = sm_cv[q];
      const int iq = sm_ci[q];
      int r = 0;
      for (int u = 0; u < nc; ++u) r += better(sm_cv[u], sm_ci[u], vq, iq) ? 1 : 0;
      if (r < width) { part_val[out0 + r] = vq; part_idx[out0 + r] = iq; }
    }
    for (int r = nc + t; r < width; r += NT) {
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
      const int i = begin + (j * NT + t) * VEC + e;
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
    for (int w = 1; w < NT / kWave; ++w)
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


// ------------------------------------------------------------------ host side

template <typename T, int WMAX, int VEC, bool ENT>
static void launch_scan(const void* logits, int vocab, int width, const ScanArgs& a,
                        hipStream_t stream) {
  const dim3 grid(a.chunks, a.rows);
  static_assert(kScanThreadsSmall * 16 == kScanThreads * 32, "both shapes cover one chunk");
  if (a.ept == 32 && static_cast<long long>(a.chunks) * a.rows <= kSmallScanGrid)
    hipLaunchKernelGGL((draft_row_scan<T, WMAX, VEC, 16, ENT, kScanThreadsSmall>), grid,
                       dim3(kScanThreadsSmall), 0, stream, static_cast<const T*>(logits), vocab,
                       a.chunks, a.chunk_len, width, a.pm, a.ps, a.pe, a.pv, a.pi, a.err);
  else if (a.ept == 32)
    hipLaunchKernelGGL((draft_row_scan<T, WMAX, VEC, 32, ENT, kScanThreads>), grid,
                       dim3(kScanThreads), 0, stream, static_cast<const T*>(logits), vocab,
                       a.chunks, a.chunk_len, width, a.pm, a.ps, a.pe, a.pv, a.pi, a.err);
  else
    hipLaunchKernelGGL((draft_row_scan<T, WMAX, VEC, 128, ENT, kScanThreads>), grid,
                       dim3(kScanThreads), 0, stream, static_cast<const T*>(logits), vocab,
                       a.chunks, a.chunk_len, width, a.pm, a.ps, a.pe, a.pv, a.pi, a.err);
}

template <typename T, int WMAX, bool ENT>
static void scan_vec(const void* logits, int vocab, int width, const ScanArgs& a,
                     hipStream_t stream) {
  constexpr int V = sizeof(T) == 4 ? 4 : 8;
  if (a.vec == V) launch_scan<T, WMAX, V, ENT>(logits, vocab, width, a, stream);
  else launch_scan<T, WMAX, 1, ENT>(logits, vocab, width, a, stream);
}

template <typename T, bool ENT>
static void scan_w(const void* logits, int vocab, int width, const ScanArgs& a,
                   hipStream_t stream) {
  switch (a.wmax) {
    case 1: scan_vec<T, 1, ENT>(logits, vocab, width, a, stream); break;
    case 2: scan_vec<T, 2, ENT>(logits, vocab, width, a, stream); break;
    case 4: scan_vec<T, 4, ENT>(logits, vocab, width, a, stream); break;
    case 8: scan_vec<T, 8, ENT>(logits, vocab, width, a, stream); break;
    default: scan_vec<T, 16, ENT>(logits, vocab, width, a, stream); break;
  }
}

hipError_t draft_scan_launch(const void* logits, jt_dtype dt, bool ent, int vocab, int width,
                             const ScanArgs& a, hipStream_t stream) {
  if (dt == JT_F32) {
    if (ent) scan_w<float, true>(logits, vocab, width, a, stream);
    else scan_w<float, false>(logits, vocab, width, a, stream);
  } else {
    if (ent) scan_w<uint16_t, true>(logits, vocab, width, a, stream);
    else scan_w<uint16_t, false>(logits, vocab, width, a, stream);
  }
  return hipGetLastError();
}

}  // namespace jt
