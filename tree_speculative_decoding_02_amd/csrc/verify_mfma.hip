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

__device__ __forceinline__ bf16x8 load16(const __bf16 *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

// 16-byte global -> LDS copy that bypasses registers (global_load_lds_dwordx4).
// Lane l's 16 bytes land at lds_wave_base + 16 * l; lds_wave_base must be
// wave-uniform.
__device__ __forceinline__ void dma16(const void *src, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(
        (__attribute__((address_space(1))) void *)(const_cast<void *>(src)),
        (__attribute__((address_space(3))) void *)lds_wave_base, 16, 0, 0);
}

// Waits until every memory operation this wave issued (DMA into LDS included) is done.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// Waits for this wave's vector-memory operations only (loads, DMA into LDS, stores);
// scalar loads and LDS operations may stay in flight.
__device__ __forceinline__ void wait_vector_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Waits until this wave's LDS reads have returned (the LDS may then be overwritten by
// DMA); vector-memory and export counters are left alone.
__device__ __forceinline__ void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Waits until at most N vector-memory operations of this wave are outstanding (they
// complete in issue order, so every older one is done); other counters are left alone.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// One wavefront per (sequence, head, 32-column slice), one workgroup per (sequence,
// head, 64-column group); the groups of one unit stay on one XCD. The kernel is
// latency-bound per wave, so it is built for occupancy: small LDS, modest registers,
// many waves in flight per SIMD. Per 32-node row tile of the tree:
//  1. Issue, back to back:
//     - Q and K fragments (16-byte loads straight into MFMA operand registers);
//     - V rows (DMA into LDS);
//     - the first two 32-row chunks of the H_0 slice (DMA into an LDS double buffer).
//  2. Topology and base-2 cumulative decay (first tile only), while the loads fly.
//  3. Intra-tree term first: S^T = K.Q^T, W, then W.V. This retires the K registers
//     early.
//  4. H_0 term, chunk by chunk: wait for chunk c (exact vmcnt), move it to registers,
//     refill its buffer with chunk c+2, then run its MFMAs.
// A second row tile (33..64 nodes) repeats the pass. Its H_0 chunks come from L2,
// and its ancestor tile-0 operands come from direct loads.
template <int DK, int DV, bool BIG>
__global__ __launch_bounds__((DV < 64 ? DV : 64) / 32 * 64, BIG ? 2 : 4) void verify_mfma_scalar_kernel(
    const float *__restrict__ H0, const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
    const __bf16 *__restrict__ v, const float *__restrict__ gate,
    const int32_t *__restrict__ parent, const int32_t *__restrict__ node_offsets,
    float *__restrict__ out, int32_t *__restrict__ tree_status, int H, int T, int U, int max_n) {
    constexpr int KS = DK / 16;                    // K-steps of Q.H0 and K.Q^T
    constexpr int NCH = DK / 32;                   // 32-row H_0 chunks (two K-steps each)
    constexpr int NW = (DV < 64 ? DV : 64) / 32;   // waves per workgroup
    constexpr int G = DV / (32 * NW);              // column groups per unit
    __shared__ float s_h0[NW][NCH][32 * 32];       // per wave: its whole H_0 slice, by 32-row chunk
    __shared__ __bf16 s_v[NW][32 * 32];            // per wave: V rows of the tile, row j at [32 j]

    const int lane = lane_id();
    const int wave = threadIdx.x >> 6;
    const int col = lane & 31, half = lane >> 5;
    int unit, cg;
    if (G == 1) {
        unit = blockIdx.x;
        cg = 0;
    } else {
        const int slot = blockIdx.x >> 3;
        cg = slot % G;
        unit = (slot / G) * 8 + (blockIdx.x & 7);
        if (unit >= U) return;
    }
    const int b = unit / H, h = unit - b * H;
    // wave-uniform column base (readfirstlane tells the compiler it is uniform, so the
    // base pointers below live in scalar registers)
    const int c0 = __builtin_amdgcn_readfirstlane((cg * NW + wave) * 32);
    const bool writer = tree_status != nullptr && h == 0 && cg == 0 && threadIdx.x == 0;

    // BIG instantiation: trees of 33..64 nodes only (everything else, status included, is
    // the small instantiation's); small instantiation: every other tree.
    const TreeRange tr = tree_range(node_offsets, b, T, BIG ? kMaxTree : max_n);
    if (BIG) {
        if (tr.status != BOLE_TREE_OK || tr.n <= 32) return;
    } else {
        if (tr.status != BOLE_TREE_OK) {
            if (writer) tree_status[b] = tr.status;
            return;
        }
        if (tr.n > 32) return;  // launched alongside the BIG instantiation
    }
    const int lo = tr.lo, n = tr.n;
    if (n == 0) {
        if (writer) tree_status[b] = BOLE_TREE_OK;
        return;
    }
    const int last = n - 1;
    // Every access below is a wave-uniform base plus a 32-bit per-lane element offset
    // (the host guarantees the offsets fit), so addresses cost one register each.
    const uint32_t rq = (uint32_t)H * DK, rv = (uint32_t)H * DV;
    const __bf16 *qu = q + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *ku = k + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *vu = v + (size_t)lo * rv + (size_t)h * DV + c0;
    float *ou = out + (size_t)lo * rv + (size_t)h * DV + c0;
    const float *hu = H0 + (size_t)unit * DK * DV + c0;

    __bf16 *lv = s_v[wave];
    // H_0 chunk c (rows 32c .. 32c+31 of the slice): instruction s moves rows 32c + 8s ..
    // +7; lane l takes row 32c + 8s + l/8, columns 4(l%8) .. +3
    const uint32_t hoff = (uint32_t)(lane >> 3) * DV + 4 * (lane & 7);
    auto dma_chunk = [&](int c, float *dst) {
#pragma unroll
        for (int s = 0; s < 4; ++s) dma16(hu + (hoff + (uint32_t)(32 * c + 8 * s) * DV), dst + 256 * s);
    };
    const uint32_t qoff_half = 8 * half;
    const uint32_t ooff = col;

    // per-node scalars first, so topology can start as soon as they land
    const int p_raw = parent[lo + min(lane, last)];
    const float g_raw = gate[(size_t)lo * H + h + (uint32_t)min(lane, last) * (uint32_t)H];

    WaveTopoL topo;
    constexpr int ntile = BIG ? 2 : 1;
    for (int it = 0; it < ntile; ++it) {
        // ---- 1. issue everything this tile needs at once: Q and K fragments (registers),
        // V rows and the whole H_0 slice (DMA into LDS). Nothing later waits on a load
        // that depends on another load.
        bf16x8 qf[KS], kf[KS];
        {
            const uint32_t qo = (uint32_t)min(32 * it + col, last) * rq + qoff_half;
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                qf[t] = load16(qu + (qo + 16 * t));
                kf[t] = load16(ku + (qo + 16 * t));
            }
        }
        {
            // V rows 32it .. 32it+31: instruction s moves 16 rows, lane l takes row
            // 32it + 16s + l/4, columns 8(l%4) .. +7 of the slice
#pragma unroll
            for (int s = 0; s < 2; ++s)
                dma16(vu + ((uint32_t)min(32 * it + 16 * s + (lane >> 2), last) * rv + 8 * (lane & 3)), lv + 512 * s);
        }
        if (it == 0) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) dma_chunk(c, s_h0[wave][c]);
        }

        // ---- 2. topology and decay, once, while the loads fly
        if (it == 0) {
            const float lg2 = lane < n ? __builtin_amdgcn_logf(g_raw) : 0.f;
            topo = wave_topology_cumlog(p_raw, lg2, n);
            if (writer) tree_status[b] = topo.bad;
            if (topo.bad) {
                wait_all_memory();  // no DMA may still target this workgroup's LDS after exit
                for (int i = half; i < n; i += 2) ou[(uint32_t)i * rv + ooff] = __builtin_nanf("");
                return;
            }
        }
        const float L2 = topo.L;  // log2 of the path's decay product, lane = node
        // Row r of accumulator element e is 32it + 8(e/4) + 4half + e%4: the same for every
        // lane of a half, so per-row values come from uniform lane reads.
        auto row_val = [&](float x, int base, int e) {
            const int r0 = base + 8 * (e >> 2) + (e & 3);
            const float v0 = readlane_f(x, r0);
            const float v1 = readlane_f(x, r0 + 4);
            return half ? v1 : v0;
        };

        // ---- 3. H0 term over the resident slice: acc = Q_it . H0 slice, H0 split into
        // bf16 hi + lo
        f32x16 acc;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] = 0.f;
        wait_all_memory();
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const float *buf = s_h0[wave][c];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 bh, bl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    __bf16 xh, xl;
                    split_bf16(buf[(16 * t + 8 * half + e) * 32 + col], xh, xl);
                    bh[e] = xh;
                    bl[e] = xl;
                }
                acc = mfma32(qf[2 * c + t], bh, acc);
                acc = mfma32(qf[2 * c + t], bl, acc);
            }
        }
        // row scale 2^{L2_i}
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[e] *= __builtin_amdgcn_exp2f(row_val(L2, 32 * it, e));

        // ---- 4. intra-tree term: ancestor tile jt = it (V from LDS), then jt = 0 for a
        // second row tile (direct loads)
        const int i = 32 * it + col;
        const uint64_t mi = shfl_u64(topo.mask, i);
        const float Li = __shfl(L2, i, 64);
        for (int jt = it; jt >= 0; --jt) {
            bf16x8 vf[2];
            const uint32_t ko = (uint32_t)min(32 * jt + col, last) * rq + qoff_half;
            if (jt == it) {
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        vf[st][e] = lv[(16 * st + 8 * (e >> 2) + 4 * half + (e & 3)) * 32 + col];
            } else {
#pragma unroll
                for (int t = 0; t < KS; ++t) kf[t] = load16(ku + (ko + 16 * t));
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        vf[st][e] = vu[(uint32_t)(32 * jt + 16 * st + 8 * (e >> 2) + 4 * half + (e & 3)) * rv + ooff];
            }
            // S^T tile: A = K rows j = 32jt + col, B = Q fragments of tile it
            f32x16 s;
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
            for (int t = 0; t < KS; ++t) s = mfma32(kf[t], qf[t], s);
            // W^T in accumulator layout: element e pairs node i with
            // j = 32jt + 8(e/4) + 4half + e%4; non-ancestors are selected to 0
            float w[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int j = 32 * jt + 8 * (e >> 2) + 4 * half + (e & 3);
                const bool anc = (mi >> j) & 1ull;
                const float d = __builtin_amdgcn_exp2f(Li - row_val(L2, 32 * jt, e));
                w[e] = anc ? s[e] * d : 0.f;
            }
            // two K-steps of 16 ancestors: element e of step st is w[8st + e], matching vf[st]
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                bf16x8 wh, wl;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    __bf16 xh, xl;
                    split_bf16(w[8 * st + e], xh, xl);
                    wh[e] = xh;
                    wl[e] = xl;
                }
                acc = mfma32(wh, vf[st], acc);
                acc = mfma32(wl, vf[st], acc);
            }
        }
        wait_lds_reads();  // this tile's LDS reads are done: the next tile may refill it

        // ---- output rows i = 32it + 8(e/4) + 4half + e%4 of column c0 + col
        if (n >= 32 * it + 32) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                ou[(uint32_t)(32 * it + 8 * (e >> 2) + 4 * half + (e & 3)) * rv + ooff] = acc[e];
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int ir = 32 * it + 8 * (e >> 2) + 4 * half + (e & 3);
                if (ir < n) ou[(uint32_t)ir * rv + ooff] = acc[e];
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
    if (a % 16 != 0) return false;
    // per-tree element offsets (64 rows of one head's rows, and one H_0 slice) are 32-bit
    const uint64_t row_elems = (uint64_t)d.heads * (uint64_t)(d.d_k > d.d_v ? d.d_k : d.d_v);
    return row_elems * kMaxTree < (1ull << 31);
}

template <int DK, int DV>
static void launch_shape(const float *H0, const __bf16 *q, const __bf16 *k, const __bf16 *v,
                         const float *gate, const int32_t *parent, const int32_t *node_offsets,
                         float *out, const bole_dims_t &d, int32_t *tree_status,
                         hipStream_t stream) {
    constexpr int NW = (DV < 64 ? DV : 64) / 32;
    constexpr int G = DV / (32 * NW);
    const unsigned U = (unsigned)d.batch * (unsigned)d.heads;
    // G > 1: ceil(U / 8) slots of 8 units, each slot G column groups wide
    const unsigned grid = G == 1 ? U : ((U + 7) / 8) * 8 * G;
    const int max_n = max_tree_nodes(d.flags);
    verify_mfma_scalar_kernel<DK, DV, false><<<dim3(grid), dim3(NW * 64), 0, stream>>>(
        H0, q, k, v, gate, parent, node_offsets, out, tree_status, d.heads, d.total_nodes,
        (int)U, max_n);
    if (max_n > 32)
        verify_mfma_scalar_kernel<DK, DV, true><<<dim3(grid), dim3(NW * 64), 0, stream>>>(
            H0, q, k, v, gate, parent, node_offsets, out, tree_status, d.heads, d.total_nodes,
            (int)U, max_n);
}

template <int DK>
static void launch_dk(const float *H0, const void *q, const void *k, const void *v,
                      const float *gate, const int32_t *parent, const int32_t *node_offsets,
                      float *out, const bole_dims_t &d, int32_t *tree_status, hipStream_t stream) {
    const __bf16 *qb = static_cast<const __bf16 *>(q), *kb = static_cast<const __bf16 *>(k),
                 *vb = static_cast<const __bf16 *>(v);
    switch (d.d_v) {
        case 32: launch_shape<DK, 32>(H0, qb, kb, vb, gate, parent, node_offsets, out, d, tree_status, stream); break;
        case 64: launch_shape<DK, 64>(H0, qb, kb, vb, gate, parent, node_offsets, out, d, tree_status, stream); break;
        case 128: launch_shape<DK, 128>(H0, qb, kb, vb, gate, parent, node_offsets, out, d, tree_status, stream); break;
        case 256: launch_shape<DK, 256>(H0, qb, kb, vb, gate, parent, node_offsets, out, d, tree_status, stream); break;
        default: break;
    }
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
