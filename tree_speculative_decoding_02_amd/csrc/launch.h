// launch.h - internal host launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bole.h"

namespace bole {

constexpr int kMaxTreeNodesHost = 64;  // nodes per tree: one wavefront, one 64-bit mask

hipError_t launch_prepare(const int32_t *parent, const int32_t *node_offsets, const float *gate,
                          const bole_dims_t &d, int32_t *depth, uint64_t *mask, float *cumlog,
                          int32_t *tree_status, hipStream_t stream);

hipError_t launch_verify_generic(const float *H0, const void *q, const void *k, const void *v,
                                 const float *gate, const int32_t *parent,
                                 const int32_t *node_offsets, float *out, const bole_dims_t &d,
                                 int32_t *tree_status, hipStream_t stream);

// True when the matrix-core verify kernel covers this request.
bool verify_mfma_applies(const bole_dims_t &d, const void *H0, const void *q, const void *k,
                         const void *v, const void *out);

hipError_t launch_verify_mfma(const float *H0, const void *q, const void *k, const void *v,
                              const float *gate, const int32_t *parent,
                              const int32_t *node_offsets, float *out, const bole_dims_t &d,
                              int32_t *tree_status, hipStream_t stream);

// True when the matrix-core vector-gate verify kernel covers this request.
bool verify_vec_applies(const bole_dims_t &d, const void *H0, const void *q, const void *k,
                        const void *v, const void *gate, const void *out);

hipError_t launch_verify_vec(const float *H0, const void *q, const void *k, const void *v,
                             const float *gate, const int32_t *parent,
                             const int32_t *node_offsets, float *out, const bole_dims_t &d,
                             int32_t *tree_status, hipStream_t stream);

// True when the one-pass lazy commit + verify kernel covers this pair of steps.
bool verify_lazy_applies(const bole_dims_t &d, const bole_dims_t &pd, const float *H0,
                         const void *q, const void *k, const void *v, const void *out,
                         const bole_factors_t &prev);

hipError_t launch_verify_lazy_commit(float *H0, const bole_factors_t &prev,
                                     const int32_t *prev_accepted_idx,
                                     const int32_t *prev_accepted_len, const bole_dims_t &pd,
                                     int32_t *prev_path_nodes, int32_t *prev_tree_status,
                                     const void *q, const void *k, const void *v,
                                     const float *gate, const int32_t *parent,
                                     const int32_t *node_offsets, float *out,
                                     const bole_dims_t &d, int32_t *tree_status,
                                     hipStream_t stream);

hipError_t launch_verify_naive(const float *H0, const void *q, const void *k, const void *v,
                               const float *gate, const int32_t *parent,
                               const int32_t *node_offsets, float *out, float *states,
                               const bole_dims_t &d, int32_t *tree_status, hipStream_t stream);

hipError_t launch_commit(float *H0, const bole_factors_t &f, const int32_t *accepted_idx,
                         const int32_t *accepted_len, const bole_dims_t &d, int32_t *path_nodes,
                         int32_t *tree_status, hipStream_t stream);

}  // namespace bole
