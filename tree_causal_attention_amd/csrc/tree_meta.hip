// jt_tree_meta: ancestor-or-self bitmask of every tree node.
//
// The tree-causal rule (JetSpec news piece, mlqm.cn/news/158889, paragraph on
// the one-forward solution; JetSpec explainer, section 三): node i sees the
// prefix, itself and its ancestors.  The mask is kept as bits -- row i, word
// w, bit b stands for tail node 32 w + b -- so the attention kernel reads a
// few words per tile instead of a dense [T, P + T] mask (the explainer's
// section 七 stages the tree mask on chip rather than expanding it densely).
//
// One workgroup per sequence; the parent array is validated and staged in LDS,
// then one thread per (row, word) walks the row's ancestor chain down to the
// word's first node (indices only decrease along the chain).
#include "jt_device.h"
#include "jt_host.h"

namespace jt {

constexpr int kMetaThreads = 1024;
constexpr int kMaxNodes = 1024;

__global__ __launch_bounds__(kMetaThreads) void tree_meta_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ n_nodes, int max_nodes,
    uint32_t* __restrict__ anc, int32_t* err) {
  static_assert(kMetaThreads >= kMaxNodes, "one thread per node slot");
  __shared__ int par[kMaxNodes];
  __shared__ int bad;
  const int seq = blockIdx.x;
  const int nw = (max_nodes + 31) / 32;
  uint32_t* out = anc + static_cast<size_t>(seq) * max_nodes * nw;
  // every slot's parent id is loaded while the node count is still in flight
  // (the array spans max_nodes per sequence); slots past the count are unused
  const int j = threadIdx.x;
  const int pj = (j < max_nodes) ? parent[static_cast<size_t>(seq) * max_nodes + j] : -1;
  const int n = n_nodes[seq];
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  if (n < 1 || n > max_nodes) {
    if (threadIdx.x == 0) report(err, JT_DERR_BAD_NNODES);
    for (int x = threadIdx.x; x < max_nodes * nw; x += kMetaThreads) out[x] = 0u;
    return;
  }
  if (j < n) {
    par[j] = pj;
    const bool ok = (j == 0) ? (pj == -1) : (pj >= 0 && pj < j);
    if (!ok) atomicOr(&bad, 1);
  }
  __syncthreads();
  if (bad) {
    if (threadIdx.x == 0) report(err, JT_DERR_BAD_PARENT);
    for (int x = threadIdx.x; x < max_nodes * nw; x += kMetaThreads) out[x] = 0u;
    return;
  }
  for (int x = threadIdx.x; x < max_nodes * nw; x += kMetaThreads) {
    const int i = x / nw, w = x % nw;
    uint32_t bits = 0u;
    if (i < n) {
      const int lo = 32 * w;
      int u = i;
      while (u >= lo) {
        if (u < lo + 32) bits |= 1u << (u - lo);
        u = par[u];
      }
    }
    out[x] = bits;
  }
}

hipError_t tree_meta_launch(const int32_t* parent, const int32_t* n_nodes, int batch,
                            int max_nodes, uint32_t* anc_mask, int32_t* err, hipStream_t stream) {
  hipLaunchKernelGGL(tree_meta_kernel, dim3(batch), dim3(kMetaThreads), 0, stream, parent, n_nodes,
                     max_nodes, anc_mask, err);
  return hipGetLastError();
}

}  // namespace jt
