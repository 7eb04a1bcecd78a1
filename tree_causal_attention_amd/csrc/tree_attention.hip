// jt_tree_attention: paged tree-causal attention of every tree node in one
// pass (JetSpec explainer, techwalker.com "加速AI思考…", section 七: paged
// tree attention with the tree mask staged on chip and the tree tail masked,
// never a dense mask; section 三: all candidate paths verified in one target
// forward; JetSpec news piece, mlqm.cn/news/158889: the tree-causal mask).
//
// bf16 path (tree_attn_mfma): one workgroup = 8 waves x 32 query rows (two
// waves per SIMD) for one (sequence, KV head, row tile, key split).  Query rows
// are (node, head of the GQA group) pairs, node-major, so every K/V tile staged
// in LDS is reused by all the group's query heads and tree nodes.
//   * The page ids of the item's key range are staged in LDS first, so tile
//     loads never wait on a page-table lookup.
//   * K and V of 4 pages (64 keys) go from global memory straight into LDS
//     (global_load_lds_dwordx4, 16 bytes per lane) into a ring of 4 stage
//     buffers; tile i+2 is fetched while tile i is computed.  Tiles are
//     row-major [key][dim] with 16-byte chunks XOR-swizzled per key (swz), so
//     the K fragment reads and the transposing V reads are bank-conflict free
//     without padding.  Explicit vmcnt waits and one barrier per tile order
//     the ring (the compiler cannot see the DMA's LDS writes).
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys as M, queries as N, so
//     each lane owns one query column and the softmax reductions stay in-lane
//     plus one cross-half exchange); Q stays in registers.
//   * Online softmax in base 2 with a lazy rescale (the running max only
//     moves when a tile exceeds it by more than 2^8).
//   * O^T += V^T P^T on the same MFMA.  P comes straight from the S^T
//     registers (the key order inside each 16-key step is permuted to match the
//     accumulator layout); the V^T operand is read from the row-major V tile
//     with ds_read_tr16_b64 transposing loads in the same key order.
// Only tiles that reach the tree tail apply the mask: the lane's node reads a
// 64-bit window of its ancestor bitmask.  Tail tiles past the row tile's last
// node are skipped (a node never sees a later node).  Work items of one
// (sequence, KV head) share an XCD; long key ranges and the small last row
// tile are split across workgroups and merged by a combine kernel.
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
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef i16x4 __attribute__((address_space(3))) * lds_i16x4_ptr;

constexpr int kKT = 64;              // keys per tile
constexpr int kWavesWG = 8;          // waves per workgroup (2 per SIMD)
constexpr int kRowsWave = 32;        // query rows per wave
constexpr int kRowsWG = kWavesWG * kRowsWave;
constexpr int kAttnThreads = kWavesWG * kWave;
constexpr int kStages = 4;           // K/V tile ring: a tile is fetched two pairs ahead
constexpr int kMaxPagesLds = 4096;   // page ids staged per work item
constexpr int kMaxTilesItem = kMaxPagesLds * kPage / kKT;
// fewest key tiles per split of a row tile: shorter splits cost more in
// per-workgroup set-up and partial rows than they gain in parallelism
constexpr int kMinTilesSplit = 4;
constexpr int kCombineWaves = 4;      // waves per merge workgroup
constexpr int kXcds = 8;             // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr double kCusPerXcd = 32.0;  // 256 CUs
constexpr double kPartialTileCost = 0.625;  // partial-tile / full-tile time per key tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (LDS and export counters left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// 16-byte chunk slot of logical chunk c of tile row `key` is c ^ swz<D>(key).
// With 256-byte rows (D = 128) a row spans all 64 banks once, so the slot is
// the bank group.  A K fragment read serves 16 lanes = 16 consecutive keys at
// one chunk per cycle: swz is a bijection on key % 16.  A transposing V read
// serves 32 lanes = 4 consecutive keys (4a..4a+3) x 4 consecutive chunks
// (4b..4b+3) per cycle: bits 2-3 of swz are key % 4 (distinct per key) and
// bits 0-1 do not depend on key % 4, so the 16 (key, chunk) pairs land on 16
// distinct slots.
template <int D>
__device__ __forceinline__ constexpr int swz(int key) {
  if constexpr (D == 128)
    return ((key & 3) << 2) | ((key >> 2) & 3);
  else
    return (((key >> 1) & 3) << 1) | ((key >> 3) & 1);  // 128-byte rows: 2 rows per bank sweep
}

// Work decomposition (identical for every (sequence, KV head) group; a
// group's actual row count and key range are read on the device):
//   rows of a group = n_nodes * group size, in row tiles of 256;
//   the rt_full full tiles are cut into s_full key splits each, the partial
//   last tile (if any) into s_part splits;
//   every group's items sit on one XCD (group sg -> XCD sg % 8) so the K/V
//   tiles its row tiles share are fetched once into that XCD's L2; within an
//   XCD the full-tile items are dealt before the cheaper partial-tile ones.
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
  _Float16* part_o;  // partial rows [ngroups * part_rows_group, D], normalised, fp16
  float* part_lse;  // [ngroups * part_rows_group]
  int32_t* err;
  int max_nodes, hq, hkv, group, max_pages, num_pages, nwords;
  int rt_full, s_full, s_part, has_partial, items_full, items_part;
  int ngroups, part_rows_group, full_part_rows;
  float scale_log2;  // scale * log2(e)
};

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

struct Item {
  int s, g, sg, rt, sp, splits;
};

// One page of zeros for the widest head (global memory, never written): K/V
// loads of pages that do not exist (past the sequence, or flagged bad) read
// it, so the loads never branch.
__device__ uint4 g_zero_page[kPage * 128 * 2 / 16];

// Maps the linear workgroup id to a work item; false for padding slots.
__device__ __forceinline__ bool decode_item(const AttnArgs& a, int L, Item& it) {
  const int xcd = L % kXcds, slot = L / kXcds;
  const int gx = (a.ngroups - xcd + kXcds - 1) / kXcds;  // groups owned by this XCD
  int j;
  if (slot < gx * a.items_full) {
    j = slot / a.items_full;
    const int i = slot % a.items_full;
    it.rt = i / a.s_full;
    it.sp = i % a.s_full;
    it.splits = a.s_full;
  } else {
    const int s2 = slot - gx * a.items_full;
    if (a.items_part == 0 || s2 >= gx * a.items_part) return false;
    j = s2 / a.items_part;
    it.rt = a.rt_full;
    it.sp = s2 % a.items_part;
    it.splits = a.s_part;
  }
  it.sg = xcd + kXcds * j;
  it.s = it.sg / a.hkv;
  it.g = it.sg % a.hkv;
  return true;
}

// Row offset of a (row tile, split) inside its group's partial block.
__device__ __forceinline__ int part_row(const AttnArgs& a, int rt, int sp) {
  if (rt < a.rt_full) return (rt * a.s_full + sp) * kRowsWG;
  return a.full_part_rows + sp * kRowsWG;
}

template <int D>
__global__ __launch_bounds__(kAttnThreads) void tree_attn_mfma(AttnArgs a) {
  constexpr int CPK = D / 8;                 // 16-byte chunks per key row
  constexpr int DB = D / 32;                 // 32-row blocks of O^T
  constexpr int KS = D / 16;                 // MFMA k-steps of K Q^T
  constexpr int TE = kKT * D;                // elements of one K (or V) tile
  constexpr int SB = 2 * TE * 2;             // bytes of one stage (K tile, then V tile)
  constexpr int IPW = kKT * CPK / kWave / kWavesWG;  // DMA instructions per wave per tensor
  static_assert(IPW * kWave * kWavesWG == kKT * CPK, "tile must split evenly over the waves");
  static_assert(kPage % (kWave * IPW / CPK) == 0, "a wave's DMA share must stay in one page");

  // Ring of kStages stage buffers (K tile, V tile); rows are unpadded and
  // XOR-swizzled at 16-byte granularity (see swz), so each DMA instruction
  // fills 1 KB of LDS contiguously.
  __shared__ __align__(1024) uint16_t stages[kStages * 2 * TE];
  __shared__ __align__(16) int pg_lds[kMaxPagesLds];

  Item item;
  if (!decode_item(a, blockIdx.x, item)) return;
  const int s = item.s, g = item.g;
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int h = lane >> 5, col = lane & 31;

  const int n = a.n_nodes[s];
  const int P = a.prefix_len[s];
  if (!seq_ok(n, P, a.max_nodes, a.max_pages, a.err,
              g == 0 && item.rt == 0 && item.sp == 0 && tid == 0))
    return;
  const int rows = n * a.group;
  const int rowbase = item.rt * kRowsWG;
  if (rowbase >= rows) return;
  const int node_hi = (min(rows, rowbase + kRowsWG) - 1) / a.group;
  const int key_end = P + node_hi + 1;  // later nodes are never visible to this tile
  const int ntiles = (key_end + kKT - 1) / kKT;
  const int tb = static_cast<int>(static_cast<long long>(ntiles) * item.sp / item.splits);
  const int te = static_cast<int>(static_cast<long long>(ntiles) * (item.sp + 1) / item.splits);
  const int nt = te - tb;

  // ---- page ids of this item's key range, staged in LDS (-1: no page)
  const int kv_len = P + n;
  const int pg0 = tb * (kKT / kPage);
  const int nslots = nt * (kKT / kPage);
  const int pg_end = (kv_len + kPage - 1) / kPage;
  {
    const int32_t* ptab = a.page_table + static_cast<size_t>(s) * a.max_pages;
    for (int i = tid; i < nslots; i += kAttnThreads) {
      int p = -1;
      if (pg0 + i < pg_end) {
        p = ptab[pg0 + i];
        if (p < 0 || p >= a.num_pages) {
          report(a.err, JT_DERR_BAD_PAGE);
          p = -1;
        }
      }
      pg_lds[i] = p;
    }
  }

  // ---- this lane's query row (B operand of K Q^T, kept in registers)
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
  // Drain the Q loads here: otherwise the wait for them lands inside the tile
  // loop and also waits for each freshly issued K/V prefetch.
  __builtin_amdgcn_s_waitcnt(0);
  const uint32_t* anc_row = a.anc + (static_cast<size_t>(s) * a.max_nodes + node) * a.nwords;
  const size_t head_stride = static_cast<size_t>(kPage) * D;
  const size_t page_stride = static_cast<size_t>(a.hkv) * head_stride;
  const uint16_t* kbase = a.k_pool + g * head_stride;
  const uint16_t* vbase = a.v_pool + g * head_stride;

  f32x16 o_acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) o_acc[db][v] = 0.0f;
  float m_run = -INFINITY;  // running max in scaled (log2) units
  float l_run = 0.0f;       // this lane's half of the normaliser

  // ---- global -> LDS directly (global_load_lds_dwordx4).  Wave w fetches
  // the chunks e = (w*IPW + i)*64 + lane of each tensor of a tile: tile row
  // e / CPK at 16-byte slot e % CPK, which holds logical chunk slot ^ swz(row);
  // a wave's rows lie in one page, so the page base is scalar.  The DMA is
  // issued through inline assembly: the compiler then does not treat every
  // LDS read as a possible reader of the stage in flight (it would wait for
  // all DMAs before each read); the explicit waits and barriers below order
  // the stages instead.
  const uint16_t* zero = reinterpret_cast<const uint16_t*>(g_zero_page);
  uint32_t dma_off[IPW];  // byte offset of the lane's chunk inside its page block
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int e = (w * IPW + i) * kWave + lane;
    const int key = e / CPK;
    dma_off[i] = ((key % kPage) * D + ((e % CPK) ^ swz<D>(key)) * 8) * 2;
  }
  const int wu = __builtin_amdgcn_readfirstlane(w);       // wave index, scalar
  const int wpage = (wu * IPW * kWave / CPK) / kPage;    // page slot of this wave's rows
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint16_t*)stages));  // LDS byte offset
  auto stage_of = [&](int ti) __attribute__((always_inline)) {
    return static_cast<uint32_t>((ti & (kStages - 1)) * SB);
  };
  auto page_of = [&](int ti) __attribute__((always_inline)) {
    return (ti < nt) ? pg_lds[ti * (kKT / kPage) + wpage] : -1;
  };
  // Issues tile ti's K and V (2*IPW instructions per wave).
  // The page id comes from a register read out of LDS one call earlier
  // (pid_next), so issuing never waits on LDS.
  int pid_next = -1;  // set once the page ids are visible
  auto issue = [&](int ti) __attribute__((always_inline)) {
    const int pid = __builtin_amdgcn_readfirstlane(pid_next);
    pid_next = page_of(ti + 1);
    const uint16_t* kp = (pid >= 0) ? kbase + static_cast<size_t>(pid) * page_stride : zero;
    const uint16_t* vp = (pid >= 0) ? vbase + static_cast<size_t>(pid) * page_stride : zero;
    const uint32_t dst = lds0 + stage_of(ti) + wu * IPW * kWave * 16;
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(dst + i * kWave * 16), "v"(dma_off[i]), "s"(kp) : "memory", "m0");
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(dst + TE * 2 + i * kWave * 16), "v"(dma_off[i]), "s"(vp)
                   : "memory", "m0");
  };
  // Keys past the sequence inside its last page hold whatever the pool holds
  // there: their scores are masked, and their V rows are zeroed here (each
  // wave clears the chunks it fetched itself, after its own DMA landed) so a
  // zero weight never meets a non-finite value.
  auto clear_v_tail = [&](int ti) __attribute__((always_inline)) {
    const int t0 = (tb + ti) * kKT;
    if (t0 + kKT <= kv_len || ti >= nt) return;
    uint16_t* vt = stages + (stage_of(ti) + TE * 2) / 2;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      const int e = (w * IPW + i) * kWave + lane;
      if (t0 + e / CPK >= kv_len) *reinterpret_cast<uint4*>(vt + e * 8) = make_uint4(0, 0, 0, 0);
    }
  };
  // LDS fragment addresses (bytes from the stage base): K fragment kk of a
  // lane is kl ^ (kk << 5); V fragment (half hf, dims block db) is
  // vl[hf] ^ (db << 6) -- XOR only touches the chunk slot bits.  Key block kb
  // adds kb*32 rows, the 16-key step ks adds 16 rows.
  const uint32_t kl = col * D * 2 + ((h ^ swz<D>(col)) << 4);
  // transposing V reads: in each 16-lane group, lane (tk, tq) points at key
  // 4h + tk (+8 for the upper half) and dims 32 db + 16 (tg&1) + 4 tq .. +3
  const int tg = lane >> 4, tk = (lane >> 2) & 3, tq = lane & 3;
  uint32_t vl[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int key = 4 * h + tk + 8 * hf;
    vl[hf] = (TE + key * D) * 2 + (((2 * (tg & 1) + (tq >> 1)) ^ swz<D>(key)) << 4) + (tq & 1) * 8;
  }

  f32x16 sacc[2];  // S^T of the tile between its QK and softmax phases
  bf16x8 pf[4];    // P^T of the tile between its softmax and PV phases
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[k][e] = static_cast<__bf16>(0.0f);

  // S^T = K Q^T for 2 blocks of 32 keys (independent accumulators interleaved)
  // (the stage base only has bits above the in-stage offset, so OR adds it;
  // the sum is made opaque per call so the compiler derives the XORed
  // fragment addresses here instead of keeping one register per fragment)
  auto qk = [&](int ti) __attribute__((always_inline)) {
    uint32_t kb_ = (lds0 + stage_of(ti)) | kl;
    asm volatile("" : "+v"(kb_));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 __attribute__((address_space(3)))*>(
            (kb_ ^ (kk << 5)) + kb * 32 * D * 2);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[kk], sacc[kb], 0, 0, 0);
      }
    }
  };

  // mask (only tiles that reach the tree tail), then online softmax in base 2
  // with a lazy rescale
  auto softmax = [&](int t0) __attribute__((always_inline)) {
    if (t0 + kKT > P) {
      const int jb = t0 - P;  // tail index of the tile's first key (may be < 0)
      const int w0 = (jb >= 0) ? (jb >> 5) : -((-jb + 31) >> 5);
      const int sh = jb - 32 * w0;  // 0..31
      uint32_t wd[3];
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int wi = w0 + k;
        wd[k] = (row_ok && wi >= 0 && wi < a.nwords) ? anc_row[wi] : 0u;
      }
      const uint64_t lo = (static_cast<uint64_t>(wd[1]) << 32) | wd[0];
      uint64_t vis = (lo >> sh) | (sh ? (static_cast<uint64_t>(wd[2]) << (64 - sh)) : 0ull);
      if (jb < 0) vis |= (1ull << -jb) - 1;  // prefix keys of a straddling tile
      // bit o of vis = key t0 + o visible; a lane's keys are o = 32 kb + 8 (v/4)
      // + 4 h + v%4, so after dropping 4 h bits each test is a constant bit.
      vis >>= 4 * h;
      const uint32_t vw[2] = {static_cast<uint32_t>(vis), static_cast<uint32_t>(vis >> 32)};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (!(vw[kb] & (1u << (8 * (v >> 2) + (v & 3))))) sacc[kb][v] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mx_s = mx * a.scale_log2;
    const bool need =
        (m_run == -INFINITY) ? (mx_s != -INFINITY) : (mx_s > m_run + kRescaleThreshold);
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? mx_s : m_run;
      const float alpha =
          need ? ((m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new)) : 1.0f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) o_acc[db][v] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    const float base = (m_run == -INFINITY) ? 0.0f : m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][v], a.scale_log2, -base));
        l_run += p;
        pf[kb * 2 + (v >> 3)][v & 7] = static_cast<__bf16>(p);
      }
  };

  // O^T += V^T P^T; V^T fragments come from the row-major V tile through
  // transposing LDS reads: in each 16-lane group, lane i gets 4 consecutive
  // keys at head dim d0 + i when its 16 lanes point at (key k, dims 4q..4q+3).
  auto pv = [&](int ti) __attribute__((always_inline)) {
    uint32_t v0 = (lds0 + stage_of(ti)) | vl[0], v1 = (lds0 + stage_of(ti)) | vl[1];
    asm volatile("" : "+v"(v0), "+v"(v1));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_ptr)((v0 ^ (db << 6)) + ks * 16 * D * 2));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4_ptr)((v1 ^ (db << 6)) + ks * 16 * D * 2));
        const uint2 ulo = __builtin_bit_cast(uint2, lo);
        const uint2 uhi = __builtin_bit_cast(uint2, hi);
        const uint4 u = make_uint4(ulo.x, ulo.y, uhi.x, uhi.y);
        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u), pf[ks],
                                                            o_acc[db], 0, 0, 0);
      }
    }
  };

  // matrix step i: O^T += V_{i-1}^T P_{i-1}^T and S_i^T = K_i Q^T.  Step 0's
  // PV reads the zeroed V tile of stage -1 with P = 0, and step nt's QK reads
  // the (zero-page) tile past the range, whose scores are never used: every
  // step runs the same code.
  auto matrix = [&](int i, int nt) __attribute__((always_inline)) {
    {
      pv(i - 1);
      qk(i);
      // Keep the LDS reads three MFMAs ahead: 48 reads (32 transposing V
      // reads, 16 K reads) feed 32 MFMAs.
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
#pragma unroll
      for (int k = 0; k < 10; ++k) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 6, 0);
    }
  };

  // Two wave groups in ping-pong: group 0 = waves 0-3, group 1 = waves 4-7,
  // one wave of each per SIMD.  A wave's steps alternate: step 2i = matrix
  // step i, step 2i+1 = softmax of tile i.  Group 0 runs step ph in phase ph,
  // group 1 runs step ph-1, so within each pair of phases group 0 does
  // [matrix i, softmax i] while group 1 does [softmax i-1, matrix i]: on every
  // SIMD one wave's MFMAs overlap the other wave's exp/max/convert work.  The
  // only barrier is at the end of each pair (one per tile), so the groups
  // drift freely inside it.
  // LDS: tile t (K_t, V_t) lives in stage t % 4.  Pair i reads K_i and
  // V_{i-1}, so tile t is read in pairs t and t+1.  At the start of pair i
  // each wave issues the DMA of tile i+2 into the stage of tile i-2 (last read
  // in pair i-1, before the barrier that closed it); at the end of pair i it
  // waits until only that DMA is in flight, so tile i+1 is complete for every
  // wave after the barrier.
  const int grp = w >> 2;
  const bool active = rowbase + w * kRowsWave < rows;  // waves with no row skip the math

  {
    // V tile of the stage read by step 0's PV (tile -1): zeros
    uint4* vz = reinterpret_cast<uint4*>(stages + (stage_of(-1) + TE * 2) / 2);
    for (int e = tid; e < TE / 8; e += kAttnThreads) vz[e] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();  // page ids and the zero tile visible
  pid_next = page_of(0);
  if (nt > 0) {
    issue(0);
    issue(1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * IPW));
    asm volatile("" ::: "memory");
    clear_v_tail(0);
    asm volatile("" ::: "memory");
  }
  __syncthreads();
#pragma unroll 1
  for (int ph = 0; ph < 2 * nt + 2; ++ph) {
    if (!(ph & 1)) issue((ph >> 1) + 2);
    const int j = ph - grp;  // this wave's step
    if (active && j >= 0 && j <= 2 * nt) {
      if ((j & 1) == 0) {
        // the wave in its matrix step wins issue arbitration against the
        // softmax of its partner on the SIMD (measured ~1% faster)
        __builtin_amdgcn_s_setprio(1);
        matrix(j >> 1, nt);
        __builtin_amdgcn_s_setprio(0);
      } else {
        softmax((tb + (j >> 1)) * kKT);
      }
    }
    if (ph & 1) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * IPW));
      asm volatile("" ::: "memory");
      clear_v_tail((ph >> 1) + 1);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
  }
  // drain the DMAs still in flight (tiles past the range) before exit
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32, kWave);
  const float inv = (l_tot > 0.0f) ? 1.0f / l_tot : 0.0f;
  const float lse_v = (l_tot > 0.0f) ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  if (!row_ok) return;
  if (item.splits == 1) {
    uint16_t* op = a.out + ((static_cast<size_t>(s) * a.max_nodes + node) * a.hq + hq) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d0 = db * 32 + 8 * grp + 4 * h;
        const __bf16 b0 = static_cast<__bf16>(o_acc[db][4 * grp + 0] * inv);
        const __bf16 b1 = static_cast<__bf16>(o_acc[db][4 * grp + 1] * inv);
        const __bf16 b2 = static_cast<__bf16>(o_acc[db][4 * grp + 2] * inv);
        const __bf16 b3 = static_cast<__bf16>(o_acc[db][4 * grp + 3] * inv);
        uint2 pk;
        pk.x = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b0)) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b1)) << 16);
        pk.y = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b2)) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b3)) << 16);
        *reinterpret_cast<uint2*>(op + d0) = pk;
      }
    if (a.lse && h == 0)
      a.lse[(static_cast<size_t>(s) * a.max_nodes + node) * a.hq + hq] = lse_v;
  } else {
    const size_t prow = static_cast<size_t>(item.sg) * a.part_rows_group +
                        part_row(a, item.rt, item.sp) + (r - rowbase);
    // a normalised partial row lies within the range of the values (|o| <=
    // max |v|): fp16 keeps it to 2^-11 relative, four times finer than the
    // bf16 output, at half the bytes of fp32 to write here and read back
    _Float16* op = a.part_o + prow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d0 = db * 32 + 8 * grp + 4 * h;
        typedef __attribute__((ext_vector_type(4))) _Float16 h4;
        h4 hv;
        hv.x = static_cast<_Float16>(o_acc[db][4 * grp] * inv);
        hv.y = static_cast<_Float16>(o_acc[db][4 * grp + 1] * inv);
        hv.z = static_cast<_Float16>(o_acc[db][4 * grp + 2] * inv);
        hv.w = static_cast<_Float16>(o_acc[db][4 * grp + 3] * inv);
        *reinterpret_cast<h4*>(op + d0) = hv;
      }
    if (h == 0) a.part_lse[prow] = lse_v;
  }
}

// Merges the per-split partials of the row tiles that were split.  A row is
// served by D / 8 lanes, each owning 8 output columns (one 16-byte load of
// fp16 per split), so a wave merges 64 / (D / 8) rows.  The lanes of a row
// spread its split log-sum-exps between them (max and weight sum by shuffles
// inside the row's lanes), then accumulate their columns over the splits with
// the loads of several splits in flight.
template <int D>
constexpr int combine_rows_per_block() { return kCombineWaves * kWave / (D / 8); }

template <int D>
__global__ __launch_bounds__(kCombineWaves * kWave) void tree_attn_combine(AttnArgs a) {
  constexpr int LPR = D / 8;                         // lanes per row
  constexpr int RPB = combine_rows_per_block<D>();   // rows per block
  constexpr int kUnroll = 8;
  static_assert(LPR % kUnroll == 0 && kWave % LPR == 0, "row lanes must tile the wave");
  typedef __attribute__((ext_vector_type(8))) _Float16 h8;
  // blocks of RPB rows: kRowsWG / RPB per split full row tile, then enough for
  // the rows of the split last row tile
  constexpr int kBlocksTile = kRowsWG / RPB;
  const int ctiles_full = a.s_full > 1 ? a.rt_full : 0;
  const int bfull = ctiles_full * kBlocksTile;
  const int lane = threadIdx.x % kWave;
  const int sl = lane % LPR, sbase = lane - sl;  // lane inside the row, first lane of the row
  const int rib = (threadIdx.x / kWave) * (kWave / LPR) + lane / LPR;  // row inside the block
  const int ctile = blockIdx.x < bfull ? blockIdx.x / kBlocksTile : ctiles_full;
  const int rloc = (blockIdx.x < bfull ? blockIdx.x % kBlocksTile : blockIdx.x - bfull) * RPB + rib;
  const int sg = blockIdx.y, s = sg / a.hkv, g = sg % a.hkv;
  const int rt = ctile < ctiles_full ? ctile : a.rt_full;
  const int splits = rt < a.rt_full ? a.s_full : a.s_part;
  const int n = a.n_nodes[s];
  const int P = a.prefix_len[s];
  if (!seq_ok(n, P, a.max_nodes, a.max_pages, a.err, false)) return;
  const int r = rt * kRowsWG + rloc;
  // every lane of a row leaves together, so the shuffles below stay inside rows
  if (r >= n * a.group) return;
  const int node = r / a.group, hq = g * a.group + r % a.group;
  const size_t gbase = static_cast<size_t>(sg) * a.part_rows_group + rloc;
  // partial row of split sp: gbase + sp0 + sp * kRowsWG
  const int sp0 = part_row(a, rt, 0);
  const float* pl = a.part_lse + gbase + sp0;
  float M = -INFINITY;
  for (int sp = sl; sp < splits; sp += LPR) M = fmaxf(M, pl[static_cast<size_t>(sp) * kRowsWG]);
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) M = fmaxf(M, shfl_xor(M, m));
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.0f;
  float wsum = 0.0f;
  for (int c0 = 0; c0 < splits; c0 += LPR) {
    // this lane's split weight (0 for splits that saw no key of the row)
    float wl = 0.0f;
    if (c0 + sl < splits) {
      const float ls = pl[static_cast<size_t>(c0 + sl) * kRowsWG];
      wl = (ls == -INFINITY) ? 0.0f : expf(ls - M);
    }
    wsum += wl;
    const int cnt = min(LPR, splits - c0);
    const _Float16* po = a.part_o + (gbase + sp0 + static_cast<size_t>(c0) * kRowsWG) * D + sl * 8;
    // kUnroll splits per round, all loads issued before the first use; slots
    // past cnt reload the last split and get weight 0 (their lanes hold 0)
    for (int k0 = 0; k0 < cnt; k0 += kUnroll) {
      h8 v[kUnroll];
#pragma unroll
      for (int kk = 0; kk < kUnroll; ++kk) {
        const int kc = min(k0 + kk, cnt - 1);
        v[kk] = *reinterpret_cast<const h8*>(po + static_cast<size_t>(kc) * kRowsWG * D);
      }
#pragma unroll
      for (int kk = 0; kk < kUnroll; ++kk) {
        const float wk = __shfl(wl, sbase + k0 + kk, kWave);
        // a zero weight contributes nothing, whatever the partial holds
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[e] += (wk != 0.0f) ? wk * static_cast<float>(v[kk][e]) : 0.0f;
      }
    }
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) wsum += shfl_xor(wsum, m);
  const float inv = 1.0f / wsum;
  uint32_t pk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    pk[k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[2 * k] * inv))) |
            (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[2 * k + 1] * inv)))
             << 16);
  uint16_t* op = a.out + ((static_cast<size_t>(s) * a.max_nodes + node) * a.hq + hq) * D;
  *reinterpret_cast<uint4*>(op + sl * 8) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  if (a.lse && sl == 0)
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
    const bool vis = t < key_end && (t < P || ((arow[(t - P) >> 5] >> ((t - P) & 31)) & 1u));
    // a bad page id is reported and its keys and values read as zero
    const float* krow = nullptr;
    if (vis) {
      const int page = ptab[t / kPage];
      if (page < 0 || page >= num_pages) report(err, JT_DERR_BAD_PAGE);
      else krow = k_pool + page * ps + g * hs + (t % kPage) * D;
    }
    float sc = -INFINITY;
    if (vis) {
      float dot = 0.0f;
      if (krow)
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
      if (page < 0 || page >= num_pages) continue;  // a zero value row adds nothing
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
  int rt_full, has_partial, s_full, s_part, ngroups, slots_per_xcd, cblocks;
  int part_rows_group, full_part_rows;
  size_t off_lse, bytes;
};

static AttnPlan attn_plan(const AttnShape& s) {
  AttnPlan p{};
  const int group = s.hq / s.hkv;
  const int rmax = s.max_nodes * group;
  p.rt_full = rmax / kRowsWG;
  p.has_partial = (rmax % kRowsWG) != 0;
  p.ngroups = s.batch * s.hkv;
  const int tiles = (s.max_pages * s.page_size + kKT - 1) / kKT;
  const int min_splits = (tiles + kMaxTilesItem - 1) / kMaxTilesItem;  // page list fits LDS
  // full tiles: enough items to fill 256 CUs once
  const long long full_items = static_cast<long long>(p.ngroups) * p.rt_full;
  int sf = full_items > 0 ? static_cast<int>((256 + full_items - 1) / full_items) : 1;
  if (full_items >= 192) sf = 1;
  const int max_splits = std::max(1, tiles / kMinTilesSplit);
  p.s_full = std::max(min_splits, std::min(sf, max_splits));
  // the partial tile has few rows: split it finely so it trails the full tiles
  int sp = static_cast<int>((256 + p.ngroups - 1) / std::max(1, p.ngroups));
  sp = std::max(sp, 4);
  p.s_part = p.has_partial ? std::max(min_splits, std::min(sp, max_splits)) : 0;
  // Few full row tiles (one or two sequences): rather than a second wave of
  // workgroups for the partial tile, fit every split of both kinds into one
  // wave of the XCD's CUs.  A partial-tile workgroup (one active wave) streams
  // a key tile in about 5/8 of a full one's time, so it gets 5/8 as many
  // splits for the same finishing time.
  if (full_items > 0 && full_items < 192 && p.has_partial) {
    const int gx = (p.ngroups + kXcds - 1) / kXcds;
    // the most full-tile splits whose items, with the partial tile's, still
    // fit the XCD's CUs once
    int sf1 = 0;
    for (int sf = 1; sf <= max_splits; ++sf) {
      const int sp = std::max(1, static_cast<int>(kPartialTileCost * sf + 0.5));
      if (gx * (p.rt_full * sf + sp) <= static_cast<int>(kCusPerXcd)) sf1 = sf;
    }
    if (sf1 >= 2) {
      const int sp1 = std::max(1, static_cast<int>(kPartialTileCost * sf1 + 0.5));
      p.s_full = std::max(min_splits, std::min(sf1, max_splits));
      p.s_part = std::max(min_splits, std::min(sp1, max_splits));
    }
  }
  const int items = p.rt_full * p.s_full + p.has_partial * p.s_part;
  const int gx_max = (p.ngroups + kXcds - 1) / kXcds;
  p.slots_per_xcd = gx_max * items;
  p.full_part_rows = p.s_full > 1 ? p.rt_full * p.s_full * kRowsWG : 0;
  p.part_rows_group = p.full_part_rows + ((p.has_partial && p.s_part > 1) ? p.s_part * kRowsWG : 0);
  // merge blocks (rb rows each): the split full row tiles, then the rows of a
  // split last row tile
  const int rb = s.head_dim == 64 ? combine_rows_per_block<64>() : combine_rows_per_block<128>();
  p.cblocks = (p.s_full > 1 ? p.rt_full * (kRowsWG / rb) : 0) +
              ((p.has_partial && p.s_part > 1) ? (rmax - p.rt_full * kRowsWG + rb - 1) / rb : 0);
  if (s.dt == JT_F32) {
    p.part_rows_group = 0;
    p.cblocks = 0;
  }
  if (p.part_rows_group > 0) {
    const size_t rows = static_cast<size_t>(p.ngroups) * p.part_rows_group;
    p.off_lse = (rows * s.head_dim * sizeof(_Float16) + 255) / 256 * 256;
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
  hipLaunchKernelGGL(tree_attn_mfma<D>, dim3(kXcds * p.slots_per_xcd), dim3(kAttnThreads), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.cblocks == 0) return e;
  hipLaunchKernelGGL(tree_attn_combine<D>, dim3(p.cblocks, p.ngroups), dim3(kCombineWaves * kWave),
                     0, stream, a);
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
  a.part_o = p.part_rows_group > 0 ? static_cast<_Float16*>(workspace) : nullptr;
  a.part_lse = p.part_rows_group > 0
                   ? reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + p.off_lse)
                   : nullptr;
  a.err = err;
  a.max_nodes = sh.max_nodes;
  a.hq = sh.hq;
  a.hkv = sh.hkv;
  a.group = sh.hq / sh.hkv;
  a.max_pages = sh.max_pages;
  a.num_pages = sh.num_pages;
  a.nwords = nwords;
  a.rt_full = p.rt_full;
  a.s_full = p.s_full;
  a.s_part = p.s_part;
  a.has_partial = p.has_partial;
  a.items_full = p.rt_full * p.s_full;
  a.items_part = p.has_partial * p.s_part;
  a.ngroups = p.ngroups;
  a.part_rows_group = p.part_rows_group;
  a.full_part_rows = p.full_part_rows;
  a.scale_log2 = scale * kLog2e;
  if (sh.head_dim == 64) return launch_mfma<64>(sh, p, a, stream);
  return launch_mfma<128>(sh, p, a, stream);
}

}  // namespace jt
