// Host-side launch entry points of the jt kernels (internal to the library;
// the public surface is include/jt.h).  Each returns the first HIP error of
// its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/jt.h"

namespace jt {

// draft_scan.hip: per-(row, chunk) partials of the draft rows
struct ScanArgs {
  int rows, chunks, chunk_len, ept, vec, wmax;
  float* pm;   // chunk max            [rows * chunks]
  double* ps;  // sum exp(x - max)     [rows * chunks]
  double* pe;  // sum exp(x - max)(x - max), only with ent
  float* pv;   // chunk top-W values   [rows * chunks * width]
  int* pi;     // chunk top-W token ids
  int32_t* err;
};
hipError_t draft_scan_launch(const void* logits, jt_dtype dt, bool ent, int vocab, int width,
                             const ScanArgs& a, hipStream_t stream);

// build_tree.hip
size_t build_tree_workspace_bytes(int batch, int depth_n, int vocab, int width);
size_t build_tree_lds_bytes(int depth_n, int width, int budget);
int build_tree_max_vocab();
hipError_t build_tree_launch(const void* logits, jt_dtype dt, int batch, int depth_n, int vocab,
                             int width, int budget, const int32_t* root_token, int32_t* parent,
                             int32_t* token, int32_t* depth, double* score, int32_t* n_nodes,
                             int32_t* err, void* workspace, hipStream_t stream);

// tree_meta.hip
hipError_t tree_meta_launch(const int32_t* parent, const int32_t* n_nodes, int batch,
                            int max_nodes, uint32_t* anc_mask, int32_t* err, hipStream_t stream);

// tree_attention.hip
struct AttnShape {
  int batch, max_nodes, hq, hkv, head_dim, max_pages, num_pages, page_size;
  jt_dtype dt;
};
size_t tree_attention_workspace_bytes(const AttnShape& s);
hipError_t tree_attention_launch(const AttnShape& s, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* n_nodes,
                                 const int32_t* prefix_len, const int32_t* page_table,
                                 const uint32_t* anc_mask, float scale, void* out, float* lse,
                                 int32_t* err, void* workspace, hipStream_t stream);

// accept.hip
size_t accept_workspace_bytes(int batch, int max_nodes, int vocab);
// no-allocation acceptance: a static device array replaces the workspace
constexpr size_t kAcceptScratchBytes = JT_ACCEPT_SCRATCH_BYTES;
hipError_t accept_scratch_address(void** out);  // this device's copy of the array
hipError_t accept_launch(const void* logits, jt_dtype dt, int batch, int max_nodes, int vocab,
                         int depth_n, const int32_t* parent, const int32_t* token,
                         const int32_t* depth, const int32_t* n_nodes, int32_t* accept_len,
                         int32_t* accept_nodes, int32_t* bonus_token, int32_t* err,
                         void* workspace, hipStream_t stream, int mode, double margin);

// stochastic.hip
hipError_t accept_stochastic_launch(const void* target, const void* draft, jt_dtype dt,
                                    int batch, int max_nodes, int vocab, int depth_n,
                                    const int32_t* parent, const int32_t* token,
                                    const int32_t* depth, const int32_t* n_nodes,
                                    float temperature, const float* u_accept,
                                    const float* u_sample, int sampled, int32_t* accept_len,
                                    int32_t* accept_nodes, int32_t* bonus_token, int32_t* err,
                                    void* workspace, hipStream_t stream);
size_t accept_stochastic_workspace_bytes(int batch, int vocab);
// build_tree.hip (variants)
hipError_t build_tree_variant_launch(const void* logits, jt_dtype dt, int batch, int depth_n,
                                     int vocab, int width, int budget, int expand_mode,
                                     double entropy_weight, const int32_t* root_token,
                                     int32_t* parent, int32_t* token, int32_t* depth,
                                     double* score, int32_t* n_nodes, int32_t* err,
                                     void* workspace, hipStream_t stream);
// commit.hip
hipError_t commit_kv_launch(void* k_pool, void* v_pool, int elem_bytes, int batch, int hkv,
                            int head_dim, const int32_t* page_table, int max_pages,
                            int num_pages, const int32_t* n_nodes, const int32_t* parent,
                            int max_nodes, int depth_n, const int32_t* accept_len,
                            const int32_t* accept_nodes, int32_t* prefix_len, int32_t* err,
                            hipStream_t stream);

}  // namespace jt
