// verify_mfma.hip - matrix-core tree verification for bf16 factors and scalar gates
// (the Mamba-2 layout).
//
// It evaluates the closed form of the Bole summary page, section 1 ("Tree-Structured
// Closed Form"), for every node of a tree at once:
//     O = diag(e^{L}) (Q H_0) + W V,   W_ij = (q_i . k_j) e^{L_i - L_j} [j on path(i)]
// L_i is the root-first sum of log a over path(i). Only per-node factors are read
// (section 2, "Token-Level Factor Encoding"); no per-node state exists anywhere.
//
// Work split: one workgroup per (sequence, head), one wavefront per 32-column slice
// of d_v. Every wavefront is self-contained:
//  - it rebuilds the tree topology on its own 64 lanes (lane = node), with no LDS and
//    no barrier;
//  - its slice of H_0 is read from HBM exactly once, straight into MFMA B-operand
//    registers;
//  - the Q and K fragments come straight from global memory in MFMA operand layout
//    (16-byte loads, since d_k is contiguous).
//
// Products, all v_mfma_f32_32x32x16_bf16 with fp32 accumulation:
//  - Q.H_0: q is bf16 already (exact). H_0 (fp32) is split into bf16 hi + lo, so two
//    passes keep about 16 mantissa bits.
//  - S^T = K.Q^T: both operands are exact bf16. The result's accumulator layout
//    (lane = column i, rows j = 8g + 4*(lane/32) + r) is reused, register for
//    register, as the A operand of W.V. This works because the contraction index j
//    may be permuted freely, as long as the V operand is gathered with the same
//    permutation. So W never goes through LDS.
//  - W.V: W is split into bf16 hi + lo (two passes). V is exact bf16.
// Masking is by select, never by multiplication, so non-ancestor pairs (whose decay
// factor may overflow) can never produce NaN.
#include "bole_device.h"
#include "launch.h"

namespace bole {

__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp32 x -> bf16 hi + bf16 lo with x ~= hi + lo (relative error about 2^-17).
__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

template <int DK, int DV>
__global__ __launch_bounds__(DV / 32 * 64) void verify_mfma_scalar_kernel(
    const float *__restrict__ H0, const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
    const __bf16 *__restrict__ v, const float *__restrict__ gate,
    const int32_t *__restrict__ parent, const int32_t *__restrict__ node_offsets,
    float *__restrict__ out, int32_t *__restrict__ tree_status, int H, int T) {
    constexpr int KS = DK / 16;  // K-steps of Q.H0 and K.Q^T
    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int unit = blockIdx.x;
    const int b = unit / H, h = unit - b * H;
    const int c0 = wave * 32;
    const bool writer = tree_status != nullptr && h == 0 && threadIdx.x == 0;

    const TreeRange tr = tree_range(node_offsets, b, T);
    if (tr.status != BOLE_TREE_OK) {
        if (writer) tree_status[b] = tr.status;
        return;
    }
    const int lo = tr.lo, n = tr.n;
    const WaveTopo topo = wave_topology(parent + lo, n);
    if (writer) tree_status[b] = topo.bad;
    if (n == 0) return;
    const size_t rq = (size_t)H * DK, rv = (size_t)H * DV;
    float *outb = out + (size_t)lo * rv + (size_t)h * DV + c0 + col;
    if (topo.bad) {
        for (int i = half; i < n; i += 2) outb[(size_t)i * rv] = __builtin_nanf("");
        return;
    }

    // Root-first cumulative log-decay, lane = node.
    const float lg = lane < n ? logf(gate[(size_t)(lo + lane) * H + h]) : 0.f;
    const float L = wave_cumlog(topo.mask, lg, n);
    const float eL = expf(L);
    const int ntile = (n + 31) >> 5;  // 32-row node tiles: 1 or 2 (wave-uniform)

    // Q fragments: lane holds node i = 32m + col, channels 16t + 8*half .. +7.
    const __bf16 *qb = q + (size_t)lo * rq + (size_t)h * DK + 8 * half;
    bf16x8 qf[2][KS];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int i = 32 * m + col;
        const bool ok = m < ntile && i < n;
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            bf16x8 z = {};
            qf[m][t] = ok ? *reinterpret_cast<const bf16x8 *>(qb + (size_t)i * rq + 16 * t) : z;
        }
    }

    // H0 term: acc[m] = Q_m . H0[:, c0 : c0 + 32], H0 split hi/lo on the fly.
    f32x16 acc[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[m][e] = 0.f;
    const float *hp = H0 + (size_t)unit * DK * DV + (size_t)(8 * half) * DV + c0 + col;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        bf16x8 bh, bl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            __bf16 xh, xl;
            split_bf16(hp[(16 * t + e) * DV], xh, xl);
            bh[e] = xh;
            bl[e] = xl;
        }
        acc[0] = mfma32(qf[0][t], bh, acc[0]);
        acc[0] = mfma32(qf[0][t], bl, acc[0]);
        if (ntile > 1) {
            acc[1] = mfma32(qf[1][t], bh, acc[1]);
            acc[1] = mfma32(qf[1][t], bl, acc[1]);
        }
    }
    // Row scale exp(L_i): accumulator element e of tile m is row i = 32m + 8(e/4) + 4half + e%4.
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        if (m < ntile) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = 32 * m + 8 * (e >> 2) + 4 * half + (e & 3);
                acc[m][e] *= __shfl(eL, i, 64);
            }
        }
    }

    // Intra-tree term, tile by tile over (node tile it, ancestor tile jt <= it).
    const __bf16 *kb = k + (size_t)lo * rq + (size_t)h * DK + 8 * half;
    const __bf16 *vb = v + (size_t)lo * rv + (size_t)h * DV + c0 + col;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        if (it >= ntile) break;
        const int i = 32 * it + col;
        const uint64_t mi = shfl_u64(topo.mask, i);
        const float Li = __shfl(L, i, 64);
#pragma unroll
        for (int jt = 0; jt <= it; ++jt) {
            // S^T tile: A = K rows j = 32jt + col, B = Q fragments of tile it.
            f32x16 s;
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = 0.f;
            const int jl = 32 * jt + col;
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                bf16x8 z = {};
                const bf16x8 kf =
                    jl < n ? *reinterpret_cast<const bf16x8 *>(kb + (size_t)jl * rq + 16 * t) : z;
                s = mfma32(kf, qf[it][t], s);
            }
            // W^T in accumulator layout: element e is pair (i, j = 32jt + 8(e/4) + 4half + e%4).
            float w[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = 32 * jt + 8 * (e >> 2) + 4 * half + (e & 3);
                const float Lj = __shfl(L, j, 64);
                const bool anc = (mi >> j) & 1ull;
                w[e] = anc ? s[e] * expf(Li - Lj) : 0.f;
            }
            // Two K-steps of 16 ancestors each. Element e of step st is w[8st + e];
            // the V operand gathers the same ancestors j in the same slots.
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                bf16x8 wh, wl, vf;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    __bf16 xh, xl;
                    split_bf16(w[8 * st + e], xh, xl);
                    wh[e] = xh;
                    wl[e] = xl;
                    const int j = 32 * jt + 16 * st + 8 * (e >> 2) + 4 * half + (e & 3);
                    vf[e] = j < n ? vb[(size_t)j * rv] : static_cast<__bf16>(0.f);
                }
                acc[it] = mfma32(wh, vf, acc[it]);
                acc[it] = mfma32(wl, vf, acc[it]);
            }
        }
    }

    // Store: element e of tile m is row i = 32m + 8(e/4) + 4half + e%4, column c0 + col.
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        if (m < ntile) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int i = 32 * m + 8 * (e >> 2) + 4 * half + (e & 3);
                if (i < n) outb[(size_t)i * rv] = acc[m][e];
            }
        }
    }
}

bool verify_mfma_applies(const bole_dims_t &d, const void *q, const void *k) {
    if (d.flags & BOLE_FLAG_FORCE_GENERIC) return false;
    if (d.factor_dtype != BOLE_DTYPE_BF16 || d.gate_kind != BOLE_GATE_SCALAR) return false;
    if (d.d_k != 64 && d.d_k != 128) return false;
    if (d.d_v != 32 && d.d_v != 64 && d.d_v != 128 && d.d_v != 256) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k);
    return (a % 16) == 0;
}

template <int DK>
static void launch_dk(const float *H0, const void *q, const void *k, const void *v,
                      const float *gate, const int32_t *parent, const int32_t *node_offsets,
                      float *out, const bole_dims_t &d, int32_t *tree_status, hipStream_t stream) {
    const dim3 grid((unsigned)d.batch * (unsigned)d.heads);
    const __bf16 *qb = static_cast<const __bf16 *>(q), *kb = static_cast<const __bf16 *>(k),
                 *vb = static_cast<const __bf16 *>(v);
#define BOLE_VERIFY_MFMA_CASE(DVV)                                                          \
    case DVV:                                                                               \
        verify_mfma_scalar_kernel<DK, DVV><<<grid, dim3(DVV / 32 * 64), 0, stream>>>(       \
            H0, qb, kb, vb, gate, parent, node_offsets, out, tree_status, d.heads,          \
            d.total_nodes);                                                                 \
        break;
    switch (d.d_v) {
        BOLE_VERIFY_MFMA_CASE(32)
        BOLE_VERIFY_MFMA_CASE(64)
        BOLE_VERIFY_MFMA_CASE(128)
        BOLE_VERIFY_MFMA_CASE(256)
        default: break;
    }
#undef BOLE_VERIFY_MFMA_CASE
}

hipError_t launch_verify_mfma(const float *H0, const void *q, const void *k, const void *v,
                              const float *gate, const int32_t *parent,
                              const int32_t *node_offsets, float *out, const bole_dims_t &d,
                              int32_t *tree_status, hipStream_t stream) {
    if (d.d_k == 64)
        launch_dk<64>(H0, q, k, v, gate, parent, node_offsets, out, d, tree_status, stream);
    else
        launch_dk<128>(H0, q, k, v, gate, parent, node_offsets, out, d, tree_status, stream);
    return hipGetLastError();
}

}  // namespace bole
