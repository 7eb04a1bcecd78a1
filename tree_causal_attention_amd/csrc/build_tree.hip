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
//   ancestors, so no deeper position can be selected).  Every position is
//   found by counting: the W candidate columns of a level are each sorted, so
//   an entry's rank in the level is its own position plus one binary search
//   per other column; its node index is its level position plus one binary
//   search per other sorted level.  Each thread owns one entry and runs its
//   searches in lockstep, so a level costs one round of searches and no merge
//   passes.  Once B kept nodes score at or above some kept score, that score
//   bounds the selection from below and later levels keep only children at or
//   above it.  All arithmetic on scores is fp64 and identical to a sequential
//   evaluation except the per-depth log-sum-exp, whose summation order
//   differs.
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

constexpr int kSelectMaxDepth = 64;

struct SelectLayout {
  int tot;     // sum of level capacities
  int capmax;  // max level capacity
  int loff[kSelectMaxDepth + 2];  // level d starts at loff[d] in the level arrays
  int coff[17];                   // column k of a level's candidates starts at coff[k]
  size_t off_S, off_lse, off_cval, off_ctok, off_loff, off_lcnt, off_npart, off_coff, off_wlen,
      off_cut, off_rawa, off_rawb;
  size_t off_canda, off_candb, off_score, off_info, off_gidx, off_order, off_ga, off_gb, off_gida,
      off_gidb, bytes;
};

inline SelectLayout select_layout(int depth_n, int width, int budget, int wmax) {
  SelectLayout L{};
  L.tot = 0;
  L.capmax = 1;
  for (int d = 1; d <= depth_n; ++d) {
    const int c = level_cap(d, width, budget);
    L.loff[d] = L.tot;
    L.tot += c;
    L.capmax = std::max(L.capmax, c);
  }
  L.loff[0] = 0;
  L.loff[depth_n + 1] = L.tot;
  // column k of a level never holds more than capmax / (k + 1) candidates
  int cc = 0;
  for (int k = 0; k < wmax; ++k) {
    L.coff[k] = cc;
    cc += std::max(1, L.capmax / (k + 1));
  }
  L.coff[wmax] = cc;
  size_t o = 0;
  auto take = [&](size_t n, size_t align) { o = (o + align - 1) / align * align; size_t r = o; o += n; return r; };
  L.off_S = take(sizeof(double) * (depth_n + 1), 8);
  L.off_lse = take(sizeof(double) * depth_n, 8);
  L.off_rawa = take(sizeof(double) * L.capmax, 8);
  L.off_rawb = take(sizeof(double) * L.capmax, 8);
  L.off_canda = take(sizeof(double) * cc, 8);
  L.off_candb = take(sizeof(double) * cc, 8);
  L.off_score = take(sizeof(double) * std::max(1, L.tot), 8);
  L.off_ga = take(sizeof(double) * std::max(1, budget), 8);
  L.off_gb = take(sizeof(double) * std::max(1, budget), 8);
  L.off_cval = take(sizeof(float) * depth_n * wmax, 4);
  L.off_ctok = take(sizeof(int) * depth_n * wmax, 4);
  L.off_loff = take(sizeof(int) * (depth_n + 2), 4);
  L.off_lcnt = take(sizeof(int) * (depth_n + 2), 4);
  L.off_npart = take(sizeof(int) * (depth_n + 2), 4);
  L.off_coff = take(sizeof(int) * 17, 4);
  L.off_wlen = take(sizeof(int) * (kSelectThreads / kWave) * wmax, 4);
  L.off_cut = take(sizeof(int) * 3 * wmax, 4);
  L.off_info = take(sizeof(uint32_t) * std::max(1, L.tot), 4);
  L.off_order = take(sizeof(uint32_t) * std::max(1, budget), 4);
  L.off_gida = take(sizeof(uint32_t) * std::max(1, budget), 4);
  L.off_gidb = take(sizeof(uint32_t) * std::max(1, budget), 4);
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

// A value every lane of the wave holds alike (read from LDS after a barrier),
// moved to scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ double uniform(double v) {
  const int2 b = __builtin_bit_cast(int2, v);
  return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readfirstlane(b.x),
                                              __builtin_amdgcn_readfirstlane(b.y)));
}

// Number of binary-search steps over n entries: ceil(log2(n + 1)).
__device__ __forceinline__ int bitwidth(int n) { return n > 0 ? 32 - __clz(n) : 0; }

// One step of a lane argmax: take the (value, id) pair a DPP lane move brings
// when it is better.  Lanes the move does not reach (row mask) keep their pair.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_better(float& v, int& id) {
  const float ov = __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, v), __builtin_bit_cast(int, v),
                                         CTRL, ROW_MASK, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(id, id, CTRL, ROW_MASK, 0xF, false);
  if (better(ov, oi, v, id)) { v = ov; id = oi; }
}

// Segmented argmax of (value, id) under `better` over SEG = 16, 32 or 64
// lanes, through DPP lane moves: quad swaps and rotations by 4 and 8 leave
// every lane of a row of 16 with the row's best; row broadcasts 15 (and 31)
// carry it into the next row (and the upper half), and the segment's last
// lane is read back (the order is total, so any combination order gives the
// same winner).
template <int SEG>
__device__ __forceinline__ void seg_best_all(float& v, int& id) {
  dpp_better<0xB1, 0xF>(v, id);   // quad_perm [1, 0, 3, 2]
  dpp_better<0x4E, 0xF>(v, id);   // quad_perm [2, 3, 0, 1]
  dpp_better<0x124, 0xF>(v, id);  // row_ror 4
  dpp_better<0x128, 0xF>(v, id);  // row_ror 8
  if constexpr (SEG >= 32) {
    dpp_better<0x142, 0xA>(v, id);  // row_bcast 15 into rows 1 and 3
    if constexpr (SEG == 64) {
      dpp_better<0x143, 0xC>(v, id);  // row_bcast 31 into rows 2 and 3
      v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
      id = __builtin_amdgcn_readlane(id, 63);
    } else {
      const bool hi = (threadIdx.x % kWave) >= 32;
      const int v31 = __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31);
      const int v63 = __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63);
      const int i31 = __builtin_amdgcn_readlane(id, 31);
      const int i63 = __builtin_amdgcn_readlane(id, 63);
      v = __builtin_bit_cast(float, hi ? v63 : v31);
      id = hi ? i63 : i31;
    }
  }
}

// Merge the chunk partials of every depth of sequence seq: one segment of SEG
// lanes a depth (SEG >= chunks; each lane holds one chunk's sorted candidates
// in registers), 64 / SEG depths a wave.  Writes lse[d], the top-W
// (cval, ctok [d * WMAX + r]) and, when part_ent is given, the entropy
// ent[d] = log S - T / S with S = sum exp(x - max), T = sum exp(x - max)(x - max).
// Lanes past `chunks` add zeros, so the sums equal those of a 64-lane
// butterfly whatever SEG is.
template <int WMAX, int SEG>
__device__ __forceinline__ void merge_depth_partials_seg(const float* __restrict__ part_max,
                                         const double* __restrict__ part_sum,
                                         const double* __restrict__ part_ent,
                                         const float* __restrict__ part_val,
                                         const int* __restrict__ part_idx, int chunks, int depth_n,
                                         int width, int seq, double* lse, double* ent,
                                         float* cval, int* ctok, int32_t* err, int nwaves) {
  constexpr int PER_WAVE = kWave / SEG;
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  const int sl = lane % SEG, sg = lane / SEG;
  for (int d0 = wv * PER_WAVE; d0 < depth_n; d0 += nwaves * PER_WAVE) {
    const int d = d0 + sg;
    const bool dok = d < depth_n;
    const size_t row = static_cast<size_t>(seq) * depth_n + (dok ? d : 0);
    const bool act = dok && sl < chunks;
    const float mc = act ? part_max[row * chunks + sl] : -INFINITY;
    const double sc = act ? part_sum[row * chunks + sl] : 0.0;
    float hv[WMAX];
    int hid[WMAX];
#pragma unroll
    for (int k = 0; k < WMAX; ++k) {
      const bool ok = act && k < width;
      hv[k] = ok ? part_val[(row * chunks + sl) * width + k] : -INFINITY;
      hid[k] = ok ? part_idx[(row * chunks + sl) * width + k] : INT32_MAX;
    }
    float M = mc;
    for (int o = SEG / 2; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, SEG));
    const double scale =
        (mc == -INFINITY) ? 0.0 : exp(static_cast<double>(mc) - static_cast<double>(M));
    double contrib = sc * scale;
    for (int o = SEG / 2; o > 0; o >>= 1) contrib += __shfl_xor(contrib, o, SEG);
    double tsum = 0.0;
    if (part_ent) {
      // the chunk's terms were taken about its own max mc: shift them to M
      const double tc = act ? part_ent[row * chunks + sl] : 0.0;
      tsum = (mc == -INFINITY)
                 ? 0.0
                 : scale * (tc + (static_cast<double>(mc) - static_cast<double>(M)) * sc);
      for (int o = SEG / 2; o > 0; o >>= 1) tsum += __shfl_xor(tsum, o, SEG);
    }
    if (sl == 0 && dok) {
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
      seg_best_all<SEG>(bv, bi);
      if (hid[0] == bi && bi != INT32_MAX) {  // this lane's head won: pop it
#pragma unroll
        for (int k = 0; k + 1 < WMAX; ++k) { hv[k] = hv[k + 1]; hid[k] = hid[k + 1]; }
        hv[WMAX - 1] = -INFINITY;
        hid[WMAX - 1] = INT32_MAX;
      }
      if (sl == 0 && dok) { cval[d * WMAX + r] = bv; ctok[d * WMAX + r] = bi; }
    }
  }
}

template <int WMAX>
__device__ __forceinline__ void merge_depth_partials(const float* __restrict__ part_max,
                                     const double* __restrict__ part_sum,
                                     const double* __restrict__ part_ent,
                                     const float* __restrict__ part_val,
                                     const int* __restrict__ part_idx, int chunks, int depth_n,
                                     int width, int seq, double* lse, double* ent, float* cval,
                                     int* ctok, int32_t* err, int nwaves) {
  if (chunks <= 16)
    merge_depth_partials_seg<WMAX, 16>(part_max, part_sum, part_ent, part_val, part_idx, chunks,
                                       depth_n, width, seq, lse, ent, cval, ctok, err, nwaves);
  else if (chunks <= 32)
    merge_depth_partials_seg<WMAX, 32>(part_max, part_sum, part_ent, part_val, part_idx, chunks,
                                       depth_n, width, seq, lse, ent, cval, ctok, err, nwaves);
  else
    merge_depth_partials_seg<WMAX, 64>(part_max, part_sum, part_ent, part_val, part_idx, chunks,
                                       depth_n, width, seq, lse, ent, cval, ctok, err, nwaves);
}

// Sum over aligned groups of N = 1, 2, 4, 8 or 16 lanes, left in every lane
// of the group, through DPP moves: quad_perm swaps within quads, then the
// half-row and row mirrors (lane i meets lane 7 - i, then 15 - i: after the
// quad sums, those pairs hold the two halves' sums).
template <int N>
__device__ __forceinline__ int group_sum(int v) {
  if constexpr (N >= 2) v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // [1,0,3,2]
  if constexpr (N >= 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // [2,3,0,1]
  if constexpr (N >= 8) v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // half mirror
  if constexpr (N >= 16) v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); // mirror
  return v;
}

struct RankArgs {
  const double* cand;    // this level's columns (column k at coff[k])
  double* cand_next;     // the next level's columns
  const double* raw_prev;
  double* raw_cur;
  double* score;         // this level's sorted scores
  uint32_t* info;        // parent position | rank << 16
  const int* coff;
  const int* wlen;        // this wave's copy of the column lengths
  const float* cv;        // this level's draft values (top-W log-probs before normalising)
  const float* cvn;       // the next level's
  int* cut_next;          // per column of the next level: first entry below tau (atomic min)
  int width, cap, cap_n;  // cap_n: the next level's capacity (0: no next level)
  double s_next;          // S of the next level
  double tau;
  int threads;
};

// Rank every candidate of a level (see phase 2 below) and place the kept
// ones.  Candidate c is served by lpc = WMAX / (KC * NG) adjacent lanes; lane
// `sub` searches the columns sub, sub + lpc, ... (KC * NG of them), KC at a
// time in lockstep.
template <int WMAX, int KC, int NG>
__device__ __forceinline__ void rank_entries(const RankArgs& a, const int (&lens)[WMAX],
                                             int items, int csteps) {
  if constexpr (KC * NG > WMAX) {
    return;
  } else {
    constexpr int LPC = WMAX / (KC * NG);
    for (int it = threadIdx.x; it < items; it += a.threads) {
      const int c = it / LPC, sub = it % LPC;
      int k = 0, p = c;
#pragma unroll
      for (int kk = 0; kk + 1 < WMAX; ++kk)
        if (k == kk && p >= lens[kk]) { p -= lens[kk]; k = kk + 1; }
      const double sc = a.cand[a.coff[k] + p];
      int cnt = 0;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        // pos[j]: the preceding prefix of column k2 found so far; steps of
        // 2^(csteps-1), ..., 1 cover any length below 2^csteps (>= m_prev)
        int pos[KC], len[KC], pt[KC];
        const double* col[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) {
          const int k2 = sub + (g * KC + j) * LPC;
          pos[j] = 0;
          len[j] = k2 != k ? a.wlen[k2] : 0;
          col[j] = a.cand + a.coff[k2] - 1;  // col[q] = entry q - 1
          pt[j] = p + (k2 < k ? 1 : 0);  // on equal scores, entry q - 1 precedes iff q <= pt
        }
        for (int half = (1 << csteps) >> 1; half > 0; half >>= 1) {
          double v[KC];
          // entry min(pos + half, len) - 1: inside the column, or for an empty
          // column the slot before it (still inside LDS, and then unused)
#pragma unroll
          for (int j = 0; j < KC; ++j) v[j] = col[j][min(pos[j] + half, len[j])];
#pragma unroll
          for (int j = 0; j < KC; ++j) {
            const int q = pos[j] + half;
            const int pr = static_cast<int>(q <= len[j]) &
                           (static_cast<int>(v[j] > sc) |
                            (static_cast<int>(v[j] == sc) & static_cast<int>(q <= pt[j])));
            pos[j] = pr ? q : pos[j];
          }
        }
#pragma unroll
        for (int j = 0; j < KC; ++j) cnt += pos[j];
      }
      cnt = group_sum<LPC>(cnt);
      const int rank = p + cnt;
      if (rank < a.cap) {
        const double raw = a.raw_prev[p] + static_cast<double>(a.cv[k]);
        if (sub == 0) {
          a.score[rank] = sc;
          a.info[rank] = static_cast<uint32_t>(p) | (static_cast<uint32_t>(k) << 16);
          a.raw_cur[rank] = raw;
        }
        // this entry's children: the next level's columns
#pragma unroll
        for (int j = 0; j < KC * NG; ++j) {
          const int k2 = sub + j * LPC;
          if (k2 < a.width && (rank + 1) * (k2 + 1) <= a.cap_n) {  // rank < cap_n / (k2 + 1)
            const double cs = (raw + static_cast<double>(a.cvn[k2])) - a.s_next;
            a.cand_next[a.coff[k2] + rank] = cs;
            if (cs < a.tau) atomicMin(&a.cut_next[k2], rank);
          }
        }
      }
    }
  }
}

// One workgroup per sequence.
//  phase 1: per depth, merge the chunk partials (lse, top-W).
//  phase 2: per level d, rank every candidate of the W columns (children of
//    the sorted level d-1 by rank k; column k cut to its first cap_d/(k+1)
//    rows) by counting; keep ranks below cap_d; update the lower bound tau.
//  phase 3: rank every kept entry across the levels under the global key; the
//    rank + 1 is the node index.
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
  double* cand_a = reinterpret_cast<double*>(smem + L.off_canda);
  double* cand_b = reinterpret_cast<double*>(smem + L.off_candb);
  double* lv_score = reinterpret_cast<double*>(smem + L.off_score);
  double* g_a = reinterpret_cast<double*>(smem + L.off_ga);
  double* g_b = reinterpret_cast<double*>(smem + L.off_gb);
  uint32_t* gid_a = reinterpret_cast<uint32_t*>(smem + L.off_gida);
  uint32_t* gid_b = reinterpret_cast<uint32_t*>(smem + L.off_gidb);
  float* cval = reinterpret_cast<float*>(smem + L.off_cval);
  int* ctok = reinterpret_cast<int*>(smem + L.off_ctok);
  int* loff = reinterpret_cast<int*>(smem + L.off_loff);
  int* lcnt = reinterpret_cast<int*>(smem + L.off_lcnt);
  int* npart = reinterpret_cast<int*>(smem + L.off_npart);
  int* coff = reinterpret_cast<int*>(smem + L.off_coff);  // column offsets (LDS copy)
  int* wlen_all = reinterpret_cast<int*>(smem + L.off_wlen);
  int* cutb = reinterpret_cast<int*>(smem + L.off_cut);  // [3][WMAX], rotating by level
  uint32_t* lv_info = reinterpret_cast<uint32_t*>(smem + L.off_info);
  uint32_t* order = reinterpret_cast<uint32_t*>(smem + L.off_order);  // node - 1 -> level << 16 | pos
  uint16_t* lv_gidx = reinterpret_cast<uint16_t*>(smem + L.off_gidx);

  const int seq = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int nwaves = kSelectThreads / kWave;

  // set-up that needs nothing from phase 1
  if (tid <= depth_n + 1) loff[tid] = L.loff[tid];
  if (tid <= WMAX) coff[tid] = L.coff[tid];
  if (tid == 0) lcnt[0] = 1;
  for (int x = tid; x < L.tot; x += kSelectThreads) lv_gidx[x] = 0xFFFF;

  // Level 1's columns (the children of the root, raw 0) and their cut at tau.
  // Reads S_1 = 0 + lse_0 and the offsets from the arguments, so pass 1 can
  // set them up in the same step as S.
  auto init_level1 = [&](int tmax, double tau0) {
    if (tid < 3 * WMAX) {
      const int k = tid % WMAX;
      const int c1 = min(L.loff[2] - L.loff[1], tmax);
      int cut = INT_MAX;
      if (k < width && k < c1) {
        const double cs = (0.0 + static_cast<double>(cval[k])) - (0.0 + lse[0]);
        if (tid < WMAX) cand_a[L.coff[k]] = cs;
        if (tid / WMAX == 1 && cs < tau0) cut = 0;
      }
      cutb[tid] = cut;
    }
    if (tid == 0) raw_a[0] = 0.0;
  };

  // ---- phase 1: merge the chunk partials of every depth
  merge_depth_partials<WMAX>(part_max, part_sum, nullptr, part_val, part_idx, chunks, depth_n,
                             width, seq, lse, nullptr, cval, ctok, err, nwaves);
  __syncthreads();
  if (tid <= depth_n) {
    // S_d = lse_0 + ... + lse_{d-1}, summed in that order
    double sd = 0.0;
    for (int j = 0; j < depth_n; ++j) {
      const double v = lse[j];
      if (j < tid) sd += v;
    }
    S[tid] = sd;
  }

  // ---- phase 2: level by level, the best children in key order.
  // The candidates of level d form W columns: column k holds the children
  // (p, k) of the first len_k parents of the sorted level d-1, with score
  // (raw_p + cval_k) - S_d (raw_p: the parent's cumulative draft log-prob
  // before normalising); a column is that sorted level shifted by one
  // constant, so it is sorted itself.  The threads that place an entry of
  // level d-1 also write its children's scores into the columns of level d.
  // An entry's rank in its level is its position p plus, for every other
  // column, the number of that column's entries that precede it, found by
  // binary search; the searches of one entry are spread over `lpc` adjacent
  // lanes (each runs its columns in lockstep, branch-free: one round trip to
  // LDS a step) and summed by lane shuffles.  Entries ranked below the level's
  // capacity are kept, written at their rank.
  //
  // tau is a lower bound of the B-th best score tau* of the tree.  Children
  // scoring below it can never be selected; in every column they form a
  // suffix, cut off before ranking, and they trail every entry >= tau in the
  // level order, so the kept levels stay prefixes of the uncut ones and the
  // result is unchanged.
  //
  // Two passes.  Pass 1 keeps at most T entries a level (the exact top T of
  // each level: the best T children of a level are children of the best T
  // parents).  Its kept entries are real nodes, so the B-th best of them,
  // tau1, is a lower bound of tau*.  It is found by merging each level into
  // G, the sorted top-B scores kept so far: one wave merges level d-1 while
  // the others rank level d, so tau lags a level behind and tightens as it
  // goes; the round after the last level merges it too.  If every level that
  // pass 1 truncated ends below tau1, no node scoring >= tau1 was left out,
  // so tau1 = tau* and the pass-1 levels hold the whole selection.  Otherwise
  // pass 2 rebuilds the levels at their full capacity, cut at tau1 from the
  // first level on.
  const int t1 = max(64, 2 * ((budget + depth_n - 1) / depth_n));
  double tau = -INFINITY;
  int last_level = 0;
  double* g_old = g_a;  // G: scores, with each entry's (level << 16 | position)
  double* g_new = g_b;
  uint32_t* gi_old = gid_a;
  uint32_t* gi_new = gid_b;
  int gn = 0;
  bool g_complete = false;  // pass 1 held the whole selection
  for (int pass = 1; pass <= 2; ++pass) {
    const bool merge_g = pass == 1;
    const int tmax = pass == 1 ? t1 : budget;
    // pass 1 leaves at least one wave to the G merge
    const int max_rank_threads = merge_g ? kSelectThreads - kWave : kSelectThreads;
    double* raw_prev = raw_a;
    double* raw_cur = raw_b;
    double* cand_cur = cand_a;
    double* cand_nxt = cand_b;
    init_level1(tmax, tau);
    __syncthreads();  // pass 1: also S and the set-up above
    int m_prev = 1;
    bool complete = true;  // pass 1: no truncated level ends at or above tau1 (checked below)
    last_level = 0;
    for (int d = 1;; ++d) {
      // level capacities are the differences of the level offsets
      const int cap_full = d <= depth_n ? uniform(loff[d + 1] - loff[d]) : 0;
      const int cap = min(cap_full, tmax);
      const bool grow = cap > 0 && m_prev > 0;
      // column lengths, cut at tau: lane k of every wave searches column k
      // column lengths: lane k of every wave holds column k's, cut where the
      // writers of the column found it drop below tau
      int* cut_cur = cutb + (d % 3) * WMAX;
      int* cut_nxt = cutb + ((d + 1) % 3) * WMAX;
      const double tau_w = tau;
      int myl = 0;
      if (grow && lane < width && lane < WMAX)
        myl = min(min(m_prev, cap / (lane + 1)), cut_cur[lane]);
      // the buffer the next round writes was last read in the previous round
      if (tid < WMAX) cutb[((d + 2) % 3) * WMAX + tid] = INT_MAX;
      // every wave keeps its own LDS copy of the column lengths (read by lane)
      if (lane < WMAX) wlen_all[(tid / kWave) * WMAX + lane] = myl;
      int lens[WMAX];
      int total_a = 0;
#pragma unroll
      for (int k = 0; k < WMAX; ++k) {
        lens[k] = __builtin_amdgcn_readlane(myl, k);
        total_a += lens[k];
      }
      const int m_d = min(cap, total_a);
      const int cap_n = (grow && d < depth_n) ? min(uniform(loff[d + 2] - loff[d + 1]), tmax) : 0;
      const double Sn = cap_n > 0 ? uniform(S[d + 1]) : 0.0;
      // lanes per entry: as many as keep every entry within one round
      int lpc = WMAX;
      while (lpc > 1 && total_a * lpc > max_rank_threads) lpc >>= 1;
      const int cpl = WMAX / lpc;  // columns per lane
      const int items = total_a * lpc;
      // the waves the ranking leaves free merge G
      const int rank_threads =
          merge_g ? min(max_rank_threads, (items + kWave - 1) / kWave * kWave) : kSelectThreads;
      const int csteps = bitwidth(m_prev);
      if (tid < rank_threads) {
        const RankArgs ra{cand_cur, cand_nxt, raw_prev, raw_cur, lv_score + loff[d],
                          lv_info + loff[d], coff, wlen_all + (tid / kWave) * WMAX,
                          cval + (d - 1) * WMAX, cap_n > 0 ? cval + d * WMAX : cval,
                          cut_nxt, width, cap, cap_n, Sn, tau_w, rank_threads};
        switch (cpl) {
          case 1: rank_entries<WMAX, 1, 1>(ra, lens, items, csteps); break;
          case 2: rank_entries<WMAX, 2, 1>(ra, lens, items, csteps); break;
          case 4: rank_entries<WMAX, 4, 1>(ra, lens, items, csteps); break;
          case 8: rank_entries<WMAX, 4, 2>(ra, lens, items, csteps); break;
          default: rank_entries<WMAX, 4, 4>(ra, lens, items, csteps); break;
        }
      } else if (merge_g && d >= 2) {
        // the remaining threads merge level d-1 into G (stable: G first on
        // equal scores), each a run of consecutive outputs found by merge path
        const int mb = m_prev;
        const double* lvl = lv_score + loff[d - 1];
        const int n_out = min(budget, gn + mb);
        const int gthreads = kSelectThreads - rank_threads;
        const int per = (n_out + gthreads - 1) / gthreads;
        const int o0 = min((tid - rank_threads) * per, n_out), o1 = min(o0 + per, n_out);
        if (o0 < o1) {
          // i = number of G entries among the first o0 outputs
          int lo = max(0, o0 - mb), hi = min(o0, gn);
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;  // does G[mid-1] come before L[o0-mid]?
            if (g_old[mid - 1] >= lvl[o0 - mid]) lo = mid; else hi = mid - 1;
          }
          int i = lo, j = o0 - lo;
          for (int o = o0; o < o1; ++o) {
            const bool take_g = i < gn && (j >= mb || g_old[i] >= lvl[j]);
            g_new[o] = take_g ? g_old[i] : lvl[j];
            gi_new[o] = take_g ? gi_old[i]
                               : (static_cast<uint32_t>(d - 1) << 16) | static_cast<uint32_t>(j);
            i += take_g ? 1 : 0;
            j += take_g ? 0 : 1;
          }
        }
      }
      __syncthreads();
      if (merge_g && d >= 2 && m_prev > 0) {
        gn = min(budget, gn + m_prev);
        double* g = g_old; g_old = g_new; g_new = g;
        uint32_t* gi = gi_old; gi_old = gi_new; gi_new = gi;
        if (gn >= budget && budget > 0) tau = uniform(g_old[budget - 1]);
      }
      if (!grow) break;
      if (tid == 0) lcnt[d] = m_d;
      if (cap < cap_full && m_d == cap) complete = false;  // truncated: checked against tau1
      double* r = raw_prev; raw_prev = raw_cur; raw_cur = r;
      double* cn = cand_cur; cand_cur = cand_nxt; cand_nxt = cn;
      m_prev = m_d;
      last_level = d;
    }
    if (pass == 2) break;
    if (complete) {
      g_complete = true;
      break;
    }
    // a full truncated level is fine when its last entry scores below tau1
    complete = true;
    for (int d0 = 1; d0 <= last_level; d0 += kWave) {
      const int d = d0 + lane;  // one level a lane
      bool bad = false;
      if (d <= last_level) {
        const int m_d = lcnt[d];
        bad = t1 < loff[d + 1] - loff[d] && m_d == t1 && !(lv_score[loff[d] + m_d - 1] < tau);
      }
      if (__ballot(bad) != 0) complete = false;
    }
    if (complete) {
      g_complete = true;
      break;
    }
    __syncthreads();  // pass 2 overwrites the levels every thread has just read
  }
  if (tid == 0)
    for (int d = last_level + 1; d <= depth_n; ++d) lcnt[d] = 0;
  // the entries scoring at least tau: a prefix of every level
  if (tid >= 1 && tid <= last_level) {
    const double* ls = lv_score + loff[tid];
    const int n = lcnt[tid];
    int lo = 0, hi = n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (ls[mid] >= tau) lo = mid + 1; else hi = mid;
    }
    npart[tid] = lo;
  }
  __syncthreads();

  // ---- phase 3: the global order.  A participant's node index is 1 + the
  // number of participants that precede it: its position in its own level
  // plus, for every other level, a binary search under the global key (ties
  // between levels compare the parents up the two paths).  The searches of
  // one participant are spread over lpc adjacent lanes, 4 levels at a time in
  // lockstep, and summed by lane shuffles.  Entries below tau trail all
  // participants and are left out.
  int tot_part = 0, maxpart = 0;
  for (int d = 1; d <= last_level; ++d) {
    const int n = npart[d];
    tot_part += n;
    maxpart = max(maxpart, n);
  }
  tot_part = uniform(tot_part);
  maxpart = uniform(maxpart);
  // When pass 1 held the selection, G is its top B in score order; with no
  // equal scores among them and no other entry at tau, that is the global
  // order itself.
  bool from_g = g_complete && gn >= budget && budget > 0 && tot_part == budget;
  if (from_g) {
    const bool tie = tid + 1 < budget && g_old[tid] == g_old[tid + 1];
    from_g = __syncthreads_or(tie) == 0;
  }
  if (from_g) {
    for (int o = tid; o < budget; o += kSelectThreads) {
      const uint32_t id = gi_old[o];
      order[o] = id;
      lv_gidx[loff[id >> 16] + (id & 0xFFFFu)] = static_cast<uint16_t>(o + 1);
    }
    tot_part = 0;  // nothing left to rank
  }
  int lpc = 16, lpc_log = 4;
  while (lpc > 1 && (tot_part * lpc > kSelectThreads || lpc / 2 >= last_level)) {
    lpc >>= 1;
    --lpc_log;
  }
  const int psteps = bitwidth(maxpart);
  for (int it = tid; it < tot_part * lpc; it += kSelectThreads) {
    const int sub = it & (lpc - 1);
    int d = 1, i = it >> lpc_log;
    while (i >= npart[d]) { i -= npart[d]; ++d; }
    const double sb = lv_score[loff[d] + i];
    int cnt = 0;
    for (int dd0 = 1 + sub; dd0 <= last_level; dd0 += 4 * lpc) {
      int lo[4], hi[4], base[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int dd = dd0 + u * lpc;
        const bool ok = dd <= last_level && dd != d;
        lo[u] = 0;
        hi[u] = ok ? npart[dd] : 0;
        base[u] = ok ? loff[dd] : 0;
      }
      for (int step = 0; step < psteps; ++step) {
        double v[4];
        // mid <= hi <= the level's length: at worst one slot past it, still
        // inside LDS, and then unused
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = lv_score[base[u] + ((lo[u] + hi[u]) >> 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int mid = (lo[u] + hi[u]) >> 1;
          const bool act = lo[u] < hi[u];
          bool pr = v[u] > sb;
          if (act && v[u] == sb)
            pr = precedes_tied(lv_score, lv_info, loff, dd0 + u * lpc, mid, d, i);
          lo[u] = (act && pr) ? mid + 1 : lo[u];
          hi[u] = (act && !pr) ? mid : hi[u];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) cnt += lo[u];
    }
    for (int o = 1; o < lpc; o <<= 1) cnt += shfl_xor(cnt, o);
    const int rank = i + cnt;
    if (sub == 0 && rank < budget) {
      order[rank] = (static_cast<uint32_t>(d) << 16) | static_cast<uint32_t>(i);
      lv_gidx[loff[d] + i] = static_cast<uint16_t>(rank + 1);
    }
  }
  const int n_sel = from_g ? budget : min(budget, tot_part);
  __syncthreads();

  // ---- phase 4: write the tree in node-index order
  const size_t base = static_cast<size_t>(seq) * (budget + 1);
  for (int o = tid; o < n_sel; o += kSelectThreads) {
    const uint32_t r = order[o];
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
