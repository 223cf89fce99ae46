// verify_vec.hip - matrix-core tree verification for bf16 factors and per-channel
// (vector) gates, the GLA / RWKV-6 layout: H_i = diag(g_i) H_parent(i) + k_i v_i^T.
//
// Closed form of the Bole summary page, section 1 ("Tree-Structured Closed Form"), with
// the diagonal transition kept per channel. With LG_i[c] = sum over path(i) of
// log2 g_m[c]:
//     o_i = H_0^T (2^{LG_i} * q_i) + sum_{j on path(i)} w_ij v_j,
//     w_ij = sum_c q_i[c] k_j[c] 2^{LG_i[c] - LG_j[c]}.
// The decay no longer factors out of the products as a row scale, so:
//  - the H_0 term runs on bf16 matrix cores with the decayed query 2^{LG_i} * q_i
//    (fp32, split hi + lo) as the A operand and H_0 (split hi + lo) as the B operand:
//    three products per tile (hi.hi, hi.lo, lo.hi);
//  - the intra-tree term touches only ancestor pairs (a node has depth-many), on the
//    vector ALU: each pair's weight is one 128-channel sum with exact exponents
//    LG_i - LG_j <= 0, so no factor can overflow.
//
// One 256-thread workgroup per (sequence, head, 64-column group), trees of up to 64
// nodes. Everything the tree needs is staged in LDS by DMA (the H_0 column slice, the
// gate, K and V rows); wavefront 0 builds the topology. Then:
//  1. gate -> log2 -> root-first cumulative sums LG, one tree level at a time;
//  2. pair weights w_ij for every ancestor pair, four lanes per node;
//  3. H_0 term, one 16-node tile per wavefront (v_mfma_f32_16x16x32_bf16), B operands
//     read from LDS as 16-byte rows (lane (n, g) takes columns 4n .. 4n+3);
//  4. the intra term accumulated into the same registers, the rows stored.
#include "bole_device.h"
#include "launch.h"
#include "mfma_util.h"

namespace bole {

constexpr int kVecThreads = 256;

template <int DK, int DV>
__global__ __launch_bounds__(kVecThreads) void verify_vec_kernel(
    const float *__restrict__ H0, const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
    const __bf16 *__restrict__ v, const float *__restrict__ gate,
    const int32_t *__restrict__ parent, const int32_t *__restrict__ node_offsets,
    float *__restrict__ out, int32_t *__restrict__ tree_status, int H, int T, int U, int max_n) {
    constexpr int N = kMaxTree;             // node rows staged (tree nodes; the rest clamped)
    constexpr int CW = DV < 64 ? DV : 64;   // state columns per workgroup
    constexpr int CPL = CW / 16;            // columns per lane in the products
    constexpr int G = DV / CW;              // column groups per unit
    constexpr int KT = DK / 32;             // k-steps of the 16x16x32 products
    constexpr int CH = DK / 4;              // channels per lane in the pair weights
    typedef float hvec __attribute__((ext_vector_type(CPL)));
    typedef __bf16 vvec __attribute__((ext_vector_type(CPL)));
    __shared__ __attribute__((aligned(16))) float s_h0[DK * CW];  // row d at [CW d]
    __shared__ __attribute__((aligned(16))) float s_lg[N * DK];   // gate -> LG, node i at [DK i]
    __shared__ __attribute__((aligned(16))) __bf16 s_k[N * DK];   // K rows
    __shared__ __attribute__((aligned(16))) __bf16 s_v[N * CW];   // V rows, the group's columns
    __shared__ float s_w[N * N];                                   // w_ij at [N i + j]
    __shared__ uint64_t s_mask[N];
    __shared__ int s_par[N], s_depth[N], s_info[2];                // info: status, max depth

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
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
    const int c0 = cg * CW;
    const bool writer = tree_status != nullptr && h == 0 && cg == 0 && tid == 0;

    const TreeRange tr = tree_range(node_offsets, b, T, max_n);
    if (tr.status != BOLE_TREE_OK) {
        if (writer) tree_status[b] = tr.status;
        return;
    }
    const int lo = tr.lo, n = tr.n;
    if (n == 0) {
        if (writer) tree_status[b] = BOLE_TREE_OK;
        return;
    }
    const int last = n - 1;
    const uint32_t rq = (uint32_t)H * DK, rv = (uint32_t)H * DV;
    const __bf16 *qu = q + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *ku = k + (size_t)lo * rq + (size_t)h * DK;
    const float *gu = gate + (size_t)lo * rq + (size_t)h * DK;
    const __bf16 *vu = v + (size_t)lo * rv + (size_t)h * DV + c0;
    float *ou = out + (size_t)lo * rv + (size_t)h * DV + c0;
    const float *hu = H0 + (size_t)unit * DK * DV + c0;

    // ---- 1. stage everything by DMA; each wavefront issues every fourth instruction.
    // A table of R rows x P 16-byte pieces moves 64/P rows per instruction; lane l takes
    // row (64/P)s + l/P, piece l%P. Node rows past the tree repeat its last row.
    {
        constexpr int HP = CW / 4;  // H_0: fp32 pieces per row
        for (int s = wave; s < DK * HP / 64; s += 4) {
            const int r = (64 / HP) * s + lane / HP;
            dma16_stream(hu + ((uint32_t)r * DV + 4 * (lane % HP)), s_h0 + 256 * s);
        }
        constexpr int GP = DK / 4;  // gate: fp32 pieces per row
        for (int s = wave; s < N * GP / 64; s += 4) {
            const int r = (64 / GP) * s + lane / GP;
            dma16_stream(gu + ((uint32_t)min(r, last) * rq + 4 * (lane % GP)), s_lg + 256 * s);
        }
        constexpr int KP = DK / 8;  // K: bf16 pieces per row
        for (int s = wave; s < N * KP / 64; s += 4) {
            const int r = (64 / KP) * s + lane / KP;
            dma16_stream(ku + ((uint32_t)min(r, last) * rq + 8 * (lane % KP)), s_k + 512 * s);
        }
        constexpr int VP = CW / 8;  // V: bf16 pieces per row
        for (int s = wave; s < N * VP / 64; s += 4) {
            const int r = (64 / VP) * s + lane / VP;
            dma16_stream(vu + ((uint32_t)min(r, last) * rv + 8 * (lane % VP)), s_v + 512 * s);
        }
    }
    // Q fragments of the H_0 term: wavefront = node tile, lane (n, g): row 16*wave + n,
    // channels 32t + 8g .. +7
    const int n16 = lane & 15, g4 = lane >> 4;
    bf16x8 qf[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t)
        qf[t] = load16_stream(qu + ((uint32_t)min(16 * wave + n16, last) * rq + 32 * t + 8 * g4));
    // query channels of the pair weights: node tid/4, channels CH*(tid%4) .. +CH-1
    const int pi = tid >> 2, psub = tid & 3;
    bf16x8 qp[CH / 8];
#pragma unroll
    for (int u = 0; u < CH / 8; ++u)
        qp[u] = load16(qu + ((uint32_t)min(pi, last) * rq + CH * psub + 8 * u));

    // ---- topology, wavefront 0
    if (wave == 0) {
        const int p = parent[lo + min(lane, last)];
        const WaveTopo topo = wave_topology_p(p, n);
        s_mask[lane] = topo.mask;
        s_par[lane] = lane < n ? p : -1;
        s_depth[lane] = topo.depth;
        // max depth over the wave: a butterfly of maxima
        int md = topo.depth;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) md = max(md, __shfl_xor(md, o, 64));
        if (lane == 0) {
            s_info[0] = topo.bad;
            s_info[1] = md;
        }
        if (writer) tree_status[b] = topo.bad;
    }
    for (int e = tid; e < N * N; e += kVecThreads) s_w[e] = 0.f;
    wait_all_memory();
    __syncthreads();

    if (s_info[0] != BOLE_TREE_OK) {
        for (int e = tid; e < n * CW; e += kVecThreads)
            ou[(uint32_t)(e / CW) * rv + (e % CW)] = __builtin_nanf("");
        return;
    }

    // ---- 2. LG: log2 of every gate entry of the tree, then root-first sums by level
    for (int e = tid; e < n * DK; e += kVecThreads) s_lg[e] = __builtin_amdgcn_logf(s_lg[e]);
    __syncthreads();
    const int max_depth = s_info[1];
    for (int d = 2; d <= max_depth; ++d) {
        for (int e = tid; e < n * DK; e += kVecThreads) {
            const int i = e / DK;
            if (s_depth[i] == d) s_lg[e] += s_lg[s_par[i] * DK + (e - i * DK)];
        }
        __syncthreads();
    }

    // ---- 3. pair weights w_ij = sum_c q_i[c] k_j[c] 2^{LG_i[c] - LG_j[c]}, j on path(i);
    // four lanes per node, CH channels each, summed across the four
    {
        const bool live = pi < n;
        const uint64_t mi = live ? s_mask[pi] : 0ull;
        float qv[CH], li[CH];
#pragma unroll
        for (int u = 0; u < CH / 8; ++u)
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[8 * u + e] = static_cast<float>(qp[u][e]);
        const float *lgi = s_lg + min(pi, last) * DK + CH * psub;
#pragma unroll
        for (int c = 0; c < CH; c += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(lgi + c);
            li[c] = x.x;
            li[c + 1] = x.y;
            li[c + 2] = x.z;
            li[c + 3] = x.w;
        }
        uint64_t rest = mi;
        while (rest) {  // the same ancestors for the four lanes of a node
            const int j = __ffsll((unsigned long long)rest) - 1;
            rest &= rest - 1;
            const float *lgj = s_lg + j * DK + CH * psub;
            const __bf16 *kj = s_k + j * DK + CH * psub;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < CH; c += 8) {
                const bf16x8 kk = *reinterpret_cast<const bf16x8 *>(kj + c);
                const float4 x0 = *reinterpret_cast<const float4 *>(lgj + c);
                const float4 x1 = *reinterpret_cast<const float4 *>(lgj + c + 4);
                const float lj[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc += qv[c + e] * static_cast<float>(kk[e]) *
                           __builtin_amdgcn_exp2f(li[c + e] - lj[e]);
            }
            acc += __shfl_xor(acc, 1, 64);
            acc += __shfl_xor(acc, 2, 64);
            if (psub == 0) s_w[pi * N + j] = acc;
        }
    }
    __syncthreads();

    // ---- 4. H_0 term for node tile `wave`: A = decayed query (hi + lo), B = H_0 rows
    // 32t + 8g + e, columns CPL*n + c (hi + lo)
    f32x4 acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int qi = min(16 * wave + n16, last);
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        const float *lgq = s_lg + qi * DK + 32 * t + 8 * g4;
        const float4 x0 = *reinterpret_cast<const float4 *>(lgq);
        const float4 x1 = *reinterpret_cast<const float4 *>(lgq + 4);
        const float lq[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        bf16x8 ah, al;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            __bf16 xh, xl;
            split_bf16(static_cast<float>(qf[t][e]) * __builtin_amdgcn_exp2f(lq[e]), xh, xl);
            ah[e] = xh;
            al[e] = xl;
        }
        bf16x8 bh[CPL], bl[CPL];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const hvec row = *reinterpret_cast<const hvec *>(s_h0 + (32 * t + 8 * g4 + e) * CW + CPL * n16);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                __bf16 xh, xl;
                split_bf16(row[c], xh, xl);
                bh[c][e] = xh;
                bl[c][e] = xl;
            }
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            acc[c] = mfma16_bf16(ah, bh[c], acc[c]);
            acc[c] = mfma16_bf16(ah, bl[c], acc[c]);
            acc[c] = mfma16_bf16(al, bh[c], acc[c]);
        }
    }

    // ---- 5. intra term into the same registers (node 16*wave + 4g + r, columns
    // CPL*n + c), then the rows
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * wave + 4 * g4 + r;
        if (i >= n) continue;
        uint64_t rest = s_mask[i];
        while (rest) {
            const int j = __ffsll((unsigned long long)rest) - 1;
            rest &= rest - 1;
            const float w = s_w[i * N + j];
            const vvec vv = *reinterpret_cast<const vvec *>(s_v + j * CW + CPL * n16);
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c][r] += w * static_cast<float>(vv[c]);
        }
        hvec o;
#pragma unroll
        for (int c = 0; c < CPL; ++c) o[c] = acc[c][r];
        __builtin_nontemporal_store(o, reinterpret_cast<hvec *>(ou + ((uint32_t)i * rv + CPL * n16)));
    }
}

bool verify_vec_applies(const bole_dims_t &d, const void *H0, const void *q, const void *k,
                        const void *v, const void *gate, const void *out) {
    if (d.flags & BOLE_FLAG_FORCE_GENERIC) return false;
    if (d.factor_dtype != BOLE_DTYPE_BF16 || d.gate_kind != BOLE_GATE_VECTOR) return false;
    if (d.d_k != 64 && d.d_k != 128) return false;
    if (d.d_v != 32 && d.d_v != 64 && d.d_v != 128 && d.d_v != 256) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(H0) | reinterpret_cast<uintptr_t>(q) |
                        reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
                        reinterpret_cast<uintptr_t>(gate) | reinterpret_cast<uintptr_t>(out);
    if (a % 16 != 0) return false;
    const uint64_t row_elems = (uint64_t)d.heads * (uint64_t)(d.d_k > d.d_v ? d.d_k : d.d_v);
    if (row_elems * kMaxTree >= (1ull << 31)) return false;
    const uint64_t groups = d.d_v > 64 ? (uint64_t)d.d_v / 64 : 1;
    return ((uint64_t)d.batch * (uint64_t)d.heads + 8) * groups < (1ull << 30);
}

template <int DK, int DV>
static void launch_vec_shape(const float *H0, const void *q, const void *k, const void *v,
                             const float *gate, const int32_t *parent,
                             const int32_t *node_offsets, float *out, const bole_dims_t &d,
                             int32_t *tree_status, hipStream_t stream) {
    constexpr int G = DV < 64 ? 1 : DV / 64;
    const unsigned U = (unsigned)d.batch * (unsigned)d.heads;
    const unsigned grid = G == 1 ? U : ((U + 7) / 8) * 8 * G;
    verify_vec_kernel<DK, DV><<<dim3(grid), dim3(kVecThreads), 0, stream>>>(
        H0, static_cast<const __bf16 *>(q), static_cast<const __bf16 *>(k),
        static_cast<const __bf16 *>(v), gate, parent, node_offsets, out, tree_status, d.heads,
        d.total_nodes, (int)U, max_tree_nodes(d.flags));
}

hipError_t launch_verify_vec(const float *H0, const void *q, const void *k, const void *v,
                             const float *gate, const int32_t *parent,
                             const int32_t *node_offsets, float *out, const bole_dims_t &d,
                             int32_t *tree_status, hipStream_t stream) {
#define BOLE_VEC_CASE(DKV, DVV)                                                                \
    if (d.d_k == DKV && d.d_v == DVV) {                                                         \
        launch_vec_shape<DKV, DVV>(H0, q, k, v, gate, parent, node_offsets, out, d, tree_status, \
                                   stream);                                                     \
        return hipGetLastError();                                                               \
    }
    BOLE_VEC_CASE(64, 32) BOLE_VEC_CASE(64, 64) BOLE_VEC_CASE(64, 128) BOLE_VEC_CASE(64, 256)
    BOLE_VEC_CASE(128, 32) BOLE_VEC_CASE(128, 64) BOLE_VEC_CASE(128, 128) BOLE_VEC_CASE(128, 256)
#undef BOLE_VEC_CASE
    return hipErrorInvalidValue;
}

}  // namespace bole
