// jt_commit_kv: moves the accepted path's tree-tail K/V rows next to the
// prefix and advances the prefix length, so the next verify step starts from
// the accepted state.  The tree tail holds node j at logical position P + j;
// the k-th accepted node a_k (depth k) moves from P + a_k to P + k; the root
// (position P) stays; the new prefix length is P + 1 + accept_len.  (JetSpec
// news piece, mlqm.cn/news/158889, tree-construction paragraph: every decode
// step starts from the hidden state the previous verification accepted.)
//
// commit_copy: one workgroup per (sequence, KV head).  Every thread first
//   loads its 16-byte chunks of all accepted rows (K and V) into registers,
//   the workgroup synchronises, then the chunks are stored at their new
//   positions: a source row may be another row's destination (a_j = k for
//   some j < k), and all reads precede all writes.
// commit_advance: prefix_len += 1 + accept_len, in a second launch so that no
//   commit_copy workgroup can read an advanced prefix length.
// Both launches run the same validation (commit_check), so a rejected
// sequence keeps its pools and its prefix length.
#include "jt_device.h"
#include "jt_host.h"

namespace jt {

constexpr int kCommitThreads = 256;
constexpr int kCommitMaxChunks = 16;  // 16-byte chunks per thread (K and V)

// Validates one sequence's commit; both launches apply the same test, so a
// sequence is either moved and advanced, or left untouched.  Returns 0 or
// the JT_DERR_* bit that rejects it:
//   BAD_PATH  n_nodes, accept_len or prefix_len out of range, accept_nodes
//             not strictly increasing in [1, n_nodes), or (with parent) not
//             the chain root -> a_1 -> ... -> a_L;
//   BAD_PAGE  a page id of a source (P + a_k) or destination (P + k) row
//             outside [0, num_pages).
__device__ __forceinline__ int commit_check(const int32_t* accept_len,
                                            const int32_t* accept_nodes, const int32_t* n_nodes,
                                            const int32_t* prefix_len, const int32_t* parent,
                                            const int32_t* page_table, int s, int max_nodes,
                                            int depth_n, int max_pages, int num_pages, int* L_out,
                                            int* P_out) {
  const int n = n_nodes[s];
  const int L = accept_len[s];
  const int P = prefix_len[s];
  if (n < 1 || n > max_nodes || L < 0 || L > depth_n || L > n - 1 || P < 0 ||
      static_cast<long long>(P) + n > static_cast<long long>(max_pages) * kPage)
    return JT_DERR_BAD_PATH;
  const int32_t* a = accept_nodes + static_cast<size_t>(s) * depth_n;
  const int32_t* par = parent ? parent + static_cast<size_t>(s) * max_nodes : nullptr;
  int prev = 0;
  for (int k = 0; k < L; ++k) {
    const int v = a[k];
    if (v <= prev || v >= n) return JT_DERR_BAD_PATH;
    if (par && par[v] != prev) return JT_DERR_BAD_PATH;
    prev = v;
  }
  // P + n <= max_pages * 16 keeps every page index below inside the table
  const int32_t* ptab = page_table + static_cast<size_t>(s) * max_pages;
  for (int k = 0; k < L; ++k) {
    const int src = ptab[(P + a[k]) / kPage], dst = ptab[(P + 1 + k) / kPage];
    if (src < 0 || src >= num_pages || dst < 0 || dst >= num_pages) return JT_DERR_BAD_PAGE;
  }
  *L_out = L;
  *P_out = P;
  return 0;
}

__global__ __launch_bounds__(kCommitThreads) void commit_copy(
    char* __restrict__ k_pool, char* __restrict__ v_pool, int row_bytes, int hkv,
    const int32_t* __restrict__ page_table, int max_pages, int num_pages,
    const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ parent, int max_nodes,
    int depth_n, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ accept_nodes, const int32_t* __restrict__ prefix_len,
    int32_t* err) {
  const int s = blockIdx.x, g = blockIdx.y;
  int L = 0, P = 0;
  const int bad = commit_check(accept_len, accept_nodes, n_nodes, prefix_len, parent, page_table,
                               s, max_nodes, depth_n, max_pages, num_pages, &L, &P);
  if (bad) {
    if (g == 0 && threadIdx.x == 0) report(err, bad);
    return;
  }
  if (L == 0) return;
  const int32_t* a = accept_nodes + static_cast<size_t>(s) * depth_n;
  const int32_t* ptab = page_table + static_cast<size_t>(s) * max_pages;
  const int cpr = row_bytes / 16;              // chunks per row
  const int total = 2 * L * cpr;               // K rows then V rows
  const size_t head_bytes = static_cast<size_t>(kPage) * row_bytes;
  const size_t page_bytes = static_cast<size_t>(hkv) * head_bytes;
  // byte address of logical position t of this sequence and head in a pool
  // (its page id was checked above)
  auto addr = [&](char* pool, int t) -> char* {
    return pool + static_cast<size_t>(ptab[t / kPage]) * page_bytes + g * head_bytes +
           static_cast<size_t>(t % kPage) * row_bytes;
  };
  uint4 buf[kCommitMaxChunks];
#pragma unroll
  for (int i = 0; i < kCommitMaxChunks; ++i) {
    const int e = threadIdx.x + i * kCommitThreads;
    if (e < total) {
      const int tensor = e / (L * cpr), r = (e / cpr) % L, c = e % cpr;
      buf[i] = reinterpret_cast<const uint4*>(addr(tensor ? v_pool : k_pool, P + a[r]))[c];
    }
  }
  __syncthreads();  // every read above precedes every write below
#pragma unroll
  for (int i = 0; i < kCommitMaxChunks; ++i) {
    const int e = threadIdx.x + i * kCommitThreads;
    if (e < total) {
      const int tensor = e / (L * cpr), r = (e / cpr) % L, c = e % cpr;
      reinterpret_cast<uint4*>(addr(tensor ? v_pool : k_pool, P + 1 + r))[c] = buf[i];
    }
  }
}

__global__ __launch_bounds__(kCommitThreads) void commit_advance(
    int batch, const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ parent,
    int max_nodes, int depth_n, const int32_t* __restrict__ page_table, int max_pages,
    int num_pages, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ accept_nodes, int32_t* __restrict__ prefix_len) {
  for (int s = blockIdx.x * kCommitThreads + threadIdx.x; s < batch;
       s += gridDim.x * kCommitThreads) {
    int L = 0, P = 0;
    if (commit_check(accept_len, accept_nodes, n_nodes, prefix_len, parent, page_table, s,
                     max_nodes, depth_n, max_pages, num_pages, &L, &P) == 0)
      prefix_len[s] = P + 1 + L;
  }
}

hipError_t commit_kv_launch(void* k_pool, void* v_pool, int elem_bytes, int batch, int hkv,
                            int head_dim, const int32_t* page_table, int max_pages,
                            int num_pages, const int32_t* n_nodes, const int32_t* parent,
                            int max_nodes, int depth_n, const int32_t* accept_len,
                            const int32_t* accept_nodes, int32_t* prefix_len, int32_t* err,
                            hipStream_t stream) {
  const int row_bytes = head_dim * elem_bytes;
  if (2 * depth_n * (row_bytes / 16) > kCommitMaxChunks * kCommitThreads)
    return hipErrorInvalidValue;  // the host entry point rejects this first
  hipLaunchKernelGGL(commit_copy, dim3(batch, hkv), dim3(kCommitThreads), 0, stream,
                     static_cast<char*>(k_pool), static_cast<char*>(v_pool), row_bytes, hkv,
                     page_table, max_pages, num_pages, n_nodes, parent, max_nodes, depth_n,
                     accept_len, accept_nodes, prefix_len, err);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int blocks = (batch + kCommitThreads - 1) / kCommitThreads;
  hipLaunchKernelGGL(commit_advance, dim3(blocks), dim3(kCommitThreads), 0, stream, batch,
                     n_nodes, parent, max_nodes, depth_n, page_table, max_pages, num_pages,
                     accept_len, accept_nodes, prefix_len);
  return hipGetLastError();
}

}  // namespace jt
