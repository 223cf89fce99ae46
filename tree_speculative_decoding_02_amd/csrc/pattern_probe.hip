// Memory-only reference kernels for the benchmark: each moves exactly the bytes of one
// tree verify (the closed form of the Bole summary page, section 1, "Tree-Structured
// Closed Form") or of one lazy step (that verify with the previous step's accepted path
// applied to H_0 first, the page's section 2 restore), in the same pieces and with a
// comparable workgroup shape, and computes nothing. The time of such a launch is what
// this access pattern costs on its own; the kernels are measured against it. Not part of
// the library's API (a separate shared object that only the benchmark loads).
//
// Scalar gates (d_k = 128, d_v = 64): per unit (sequence, head) the 32 KB H_0 slice, the
// tree's q and k rows (256-byte pieces, rows H * 256 bytes apart), v rows (128 bytes) and
// gate scalars are read, then the out rows (256 bytes) written; 128 threads per unit, NU
// units (neighbouring heads) per workgroup.
// Vector gates (d_k = d_v = 128): per unit the 64 KB H_0 slice, the tree's gate rows
// (512-byte pieces), k, q and v rows (256 bytes) are read and the out rows (512 bytes)
// written; one 512-thread workgroup per unit.
//
// Every load is issued before the first is used; the values are folded into one register
// and stored as the output rows, so no load can be dropped.
#include <hip/hip_runtime.h>

#include <cstdint>

#define PROBE_API extern "C" __attribute__((visibility("default")))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Tree {
    int lo, n;
};

// the sequence's tree, or n = 0 when its offsets are not a tree of 1..64 nodes in [0, T)
__device__ __forceinline__ Tree tree_of(const int32_t *offs, int b, int T) {
    const int lo = offs[b], hi = offs[b + 1];
    const bool ok = lo >= 0 && hi > lo && hi <= T && hi - lo <= 64;
    return Tree{lo, ok ? hi - lo : 0};
}

template <int NU>
__global__ __launch_bounds__(128 * NU) void scalar_traffic(const float *__restrict__ H0,
                                                           const uint16_t *__restrict__ q,
                                                           const uint16_t *__restrict__ k,
                                                           const uint16_t *__restrict__ v,
                                                           const float *__restrict__ gate,
                                                           float *__restrict__ out,
                                                           const int32_t *__restrict__ offs,
                                                           int H, int U, int T) {
    constexpr int DK = 128, DV = 64;
    const int tid = threadIdx.x & 127;
    const int unit = NU * (int)blockIdx.x + (int)(threadIdx.x >> 7);
    if (unit >= U) return;
    const int b = unit / H, h = unit - b * H;
    const Tree tr = tree_of(offs, b, T);
    if (tr.n == 0) return;
    const int n = tr.n;
    const uint32_t rq = (uint32_t)H * DK, rv = (uint32_t)H * DV;
    const uint16_t *qu = q + (size_t)tr.lo * rq + (size_t)h * DK;
    const uint16_t *ku = k + (size_t)tr.lo * rq + (size_t)h * DK;
    const uint16_t *vu = v + (size_t)tr.lo * rv + (size_t)h * DV;
    const float *hu = H0 + (size_t)unit * DK * DV;
    u32x4 r[37];
#pragma unroll
    for (int u = 0; u < 16; ++u)  // H_0: 2048 pieces of 16 bytes
        r[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(hu + 4 * (tid + 128 * u)));
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // q and k: 16 pieces per row, the tree's rows only
        const int p = tid + 128 * u;
        r[16 + u] = u32x4{0u, 0u, 0u, 0u};
        r[24 + u] = u32x4{0u, 0u, 0u, 0u};
        if (p / 16 < n) {
            r[16 + u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(qu + (uint32_t)(p / 16) * rq + 8 * (p % 16)));
            r[24 + u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(ku + (uint32_t)(p / 16) * rq + 8 * (p % 16)));
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // v: 8 pieces per row
        const int p = tid + 128 * u;
        r[32 + u] = u32x4{0u, 0u, 0u, 0u};
        if (p / 8 < n)
            r[32 + u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(vu + (uint32_t)(p / 8) * rv + 8 * (p % 8)));
    }
    const float gv = tid < n ? gate[(size_t)(tr.lo + tid) * H + h] : 0.f;
    r[36] = u32x4{__float_as_uint(gv), 0u, 0u, 0u};
    u32x4 acc = r[0];
#pragma unroll
    for (int u = 1; u < 37; ++u) acc ^= r[u];
    float *ou = out + (size_t)tr.lo * rv + (size_t)h * DV;
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // out: 16 pieces per row
        const int p = tid + 128 * u;
        if (p / 16 < n)
            __builtin_nontemporal_store(
                acc, reinterpret_cast<u32x4 *>(ou + (uint32_t)(p / 16) * rv + 4 * (p % 16)));
    }
}

__global__ __launch_bounds__(512) void vector_traffic(const float *__restrict__ H0,
                                                      const uint16_t *__restrict__ q,
                                                      const uint16_t *__restrict__ k,
                                                      const uint16_t *__restrict__ v,
                                                      const float *__restrict__ gate,
                                                      float *__restrict__ out,
                                                      const int32_t *__restrict__ offs, int H,
                                                      int T) {
    constexpr int DK = 128, DV = 128, NT = 512;
    const int unit = blockIdx.x, b = unit / H, h = unit - b * H, tid = threadIdx.x;
    const Tree tr = tree_of(offs, b, T);
    if (tr.n == 0) return;
    const int n = tr.n, last = n - 1;
    const uint32_t rq = (uint32_t)H * DK, rv = (uint32_t)H * DV;
    const float *gu = gate + (size_t)tr.lo * rq + (size_t)h * DK;
    const uint16_t *ku = k + (size_t)tr.lo * rq + (size_t)h * DK;
    const uint16_t *qu = q + (size_t)tr.lo * rq + (size_t)h * DK;
    const uint16_t *vu = v + (size_t)tr.lo * rv + (size_t)h * DV;
    const float *hu = H0 + (size_t)unit * DK * DV;
    u32x4 r[18];
    // rows past the tree repeat its last row, as the verify's staging does
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // gate: 32 pieces per row
        const int p = tid + NT * u;
        r[u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(gu + (uint32_t)min(p / 32, last) * rq + 4 * (p % 32)));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // k and q: 16 pieces per row
        const int p = tid + NT * u;
        r[4 + u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(ku + (uint32_t)min(p / 16, last) * rq + 8 * (p % 16)));
        r[6 + u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(qu + (uint32_t)min(p / 16, last) * rq + 8 * (p % 16)));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // H_0: 4096 pieces
        const int p = tid + NT * u;
        r[8 + u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(hu + 4 * p));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // v: 16 pieces per row
        const int p = tid + NT * u;
        r[16 + u] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4 *>(vu + (uint32_t)min(p / 16, last) * rv + 8 * (p % 16)));
    }
    u32x4 acc = r[0];
#pragma unroll
    for (int u = 1; u < 18; ++u) acc ^= r[u];
    float *ou = out + (size_t)tr.lo * rv + (size_t)h * DV;
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // out: 32 pieces per row
        const int p = tid + NT * u;
        if (p / 32 < n)
            __builtin_nontemporal_store(
                acc, reinterpret_cast<u32x4 *>(ou + (uint32_t)(p / 32) * rv + 4 * (p % 32)));
    }
}

// One layer of the lazy step: the state and factors of this step's tree and the previous
// step's path factors (each layer its own).
struct ProbeLayer {
    float *H0;
    const uint16_t *q, *k, *v;
    const float *gate;
    float *out;
    const uint16_t *prev_k, *prev_v;
    const float *prev_gate;
};
constexpr int kProbeLayers = 16;
struct ProbeTable {
    ProbeLayer l[kProbeLayers];
};

// Lazy-step traffic (d_k = 128, d_v = 64): per unit the 32 KB H_0 slice read, the path's
// k and v rows (256- and 128-byte pieces) and gate scalars read, H_0 written back (the
// values read, so the state is unchanged) when the path is not empty, then the tree's
// rows as scalar_traffic. 128 threads per unit, two units per workgroup, blockIdx.y =
// layer.
__global__ __launch_bounds__(256) void lazy_traffic(const ProbeTable t,
                                                    const int32_t *__restrict__ offs,
                                                    const int32_t *__restrict__ poffs,
                                                    const int32_t *__restrict__ acc_idx,
                                                    const int32_t *__restrict__ acc_len,
                                                    int max_path, int H, int U, int T, int PT) {
    constexpr int DK = 128, DV = 64, PPN = 24;  // path pieces per node: 16 of k, 8 of v
    const ProbeLayer &ly = t.l[blockIdx.y];
    const int tid = threadIdx.x & 127;
    const int unit = 2 * (int)blockIdx.x + (int)(threadIdx.x >> 7);
    if (unit >= U) return;
    const int b = unit / H, h = unit - b * H;
    const Tree tr = tree_of(offs, b, T);
    const Tree pt = tree_of(poffs, b, PT);
    const int L0 = acc_len[b];
    const int L = (pt.n > 0 && L0 > 0 && L0 <= max_path && L0 <= pt.n) ? L0 : 0;
    const int32_t *ai = acc_idx + (size_t)b * max_path;
    const uint32_t rq = (uint32_t)H * DK, rv = (uint32_t)H * DV;
    float *hu = ly.H0 + (size_t)unit * DK * DV;
    u32x4 hr[16], r[33];
#pragma unroll
    for (int u = 0; u < 16; ++u)  // H_0
        hr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(hu + 4 * (tid + 128 * u)));
#pragma unroll
    for (int u = 0; u < 12; ++u) {  // the path's k and v pieces
        const int p = tid + 128 * u, m = p / PPN, part = p % PPN;
        r[u] = u32x4{0u, 0u, 0u, 0u};
        if (m < L) {
            const int x = ai[m];
            if (x >= 0 && x < pt.n) {
                const size_t row = (size_t)(pt.lo + x) * H + h;
                r[u] = part < 16
                           ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ly.prev_k + row * DK + 8 * part))
                           : __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(ly.prev_v + row * DV + 8 * (part - 16)));
            }
        }
    }
    float pg = 0.f;
    if (tid < L) {
        const int x = ai[tid];
        if (x >= 0 && x < pt.n) pg = ly.prev_gate[(size_t)(pt.lo + x) * H + h];
    }
    const int n = tr.n;
    const uint16_t *qu = ly.q + (size_t)tr.lo * rq + (size_t)h * DK;
    const uint16_t *ku = ly.k + (size_t)tr.lo * rq + (size_t)h * DK;
    const uint16_t *vu = ly.v + (size_t)tr.lo * rv + (size_t)h * DV;
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // q and k: 16 pieces per row
        const int p = tid + 128 * u;
        r[12 + u] = u32x4{0u, 0u, 0u, 0u};
        r[20 + u] = u32x4{0u, 0u, 0u, 0u};
        if (p / 16 < n) {
            r[12 + u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(qu + (uint32_t)(p / 16) * rq + 8 * (p % 16)));
            r[20 + u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(ku + (uint32_t)(p / 16) * rq + 8 * (p % 16)));
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // v: 8 pieces per row
        const int p = tid + 128 * u;
        r[28 + u] = u32x4{0u, 0u, 0u, 0u};
        if (p / 8 < n)
            r[28 + u] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4 *>(vu + (uint32_t)(p / 8) * rv + 8 * (p % 8)));
    }
    const float gv = tid < n ? ly.gate[(size_t)(tr.lo + tid) * H + h] : 0.f;
    r[32] = u32x4{__float_as_uint(gv), __float_as_uint(pg), 0u, 0u};
    if (L > 0) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            // the values read, made opaque to the compiler: a store of a value just loaded
            // from the same address would otherwise be dropped as a no-op
            u32x4 x = hr[u];
            asm volatile("" : "+v"(x));
            __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(hu + 4 * (tid + 128 * u)));
        }
    }
    u32x4 acc = hr[0];
#pragma unroll
    for (int u = 1; u < 16; ++u) acc ^= hr[u];
#pragma unroll
    for (int u = 0; u < 33; ++u) acc ^= r[u];
    float *ou = ly.out + (size_t)tr.lo * rv + (size_t)h * DV;
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // out: 16 pieces per row
        const int p = tid + 128 * u;
        if (p / 16 < n)
            __builtin_nontemporal_store(
                acc, reinterpret_cast<u32x4 *>(ou + (uint32_t)(p / 16) * rv + 4 * (p % 16)));
    }
}

// Lazy-step traffic with per-channel gates (d_k = d_v = 128), in the vector-gate kernel's
// lazy launch shape: one 256-thread workgroup per (unit, 64-column group), the two groups
// of a unit 8 workgroups apart (slots of 8 units). Each reads its 32 KB half of the H_0
// slice, the path's gate and k rows and its half of their v rows, and the tree's gate, q and
// k rows and its half of the v rows; it writes its H_0 half back (the values read) when the
// path is not empty, then its half of the out rows. The rows both groups read take plain
// loads, as in the kernel, so the second read can come from L2. blockIdx.y = layer.
__global__ __launch_bounds__(256) void vector_lazy_traffic(const ProbeTable t,
                                                           const int32_t *__restrict__ offs,
                                                           const int32_t *__restrict__ poffs,
                                                           const int32_t *__restrict__ acc_idx,
                                                           const int32_t *__restrict__ acc_len,
                                                           int max_path, int H, int U, int T, int PT) {
    constexpr int DK = 128, DV = 128, CW = 64, NT = 256;
    constexpr int PPN = DK / 4 + DK / 8 + CW / 8;  // path pieces per node: gate, k, v half
    const ProbeLayer &ly = t.l[blockIdx.y];
    const int tid = threadIdx.x;
    const int slot = blockIdx.x >> 3, cg = slot & 1;
    const int unit = (slot >> 1) * 8 + (blockIdx.x & 7);
    if (unit >= U) return;
    const int b = unit / H, h = unit - b * H;
    const int c0 = cg * CW;
    const Tree tr = tree_of(offs, b, T);
    const Tree pt = tree_of(poffs, b, PT);
    const int L0 = acc_len[b];
    const int L = (pt.n > 0 && L0 > 0 && L0 <= max_path && L0 <= pt.n) ? L0 : 0;
    const int32_t *ai = acc_idx + (size_t)b * max_path;
    const uint32_t rq = (uint32_t)H * DK, rv = (uint32_t)H * DV;
    float *hu = ly.H0 + (size_t)unit * DK * DV + c0;
    u32x4 hr[8], r[18];
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // the H_0 half: row p / 16, piece p % 16
        const int p = tid + NT * u;
        hr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(hu + (uint32_t)(p / 16) * DV + 4 * (p % 16)));
    }
    u32x4 pacc = u32x4{0u, 0u, 0u, 0u};
    for (int p = tid; p < L * PPN; p += NT) {  // the path's pieces
        const int m = p / PPN, part = p % PPN;
        const int x = ai[m];
        if (x >= 0 && x < pt.n) {
            const size_t row = (size_t)(pt.lo + x) * H + h;
            pacc ^= part < DK / 4
                        ? *reinterpret_cast<const u32x4 *>(ly.prev_gate + row * DK + 4 * part)
                    : part < DK / 4 + DK / 8
                        ? *reinterpret_cast<const u32x4 *>(ly.prev_k + row * DK + 8 * (part - DK / 4))
                        : __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                              ly.prev_v + row * DV + c0 + 8 * (part - DK / 4 - DK / 8)));
        }
    }
    const int n = tr.n;
    const float *gu = ly.gate + (size_t)tr.lo * rq + (size_t)h * DK;
    const uint16_t *qu = ly.q + (size_t)tr.lo * rq + (size_t)h * DK;
    const uint16_t *ku = ly.k + (size_t)tr.lo * rq + (size_t)h * DK;
    const uint16_t *vu = ly.v + (size_t)tr.lo * rv + (size_t)h * DV + c0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // gate: 32 pieces per row
        const int p = tid + NT * u;
        r[u] = p / 32 < n ? *reinterpret_cast<const u32x4 *>(gu + (uint32_t)(p / 32) * rq + 4 * (p % 32))
                          : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // q and k: 16 pieces per row
        const int p = tid + NT * u;
        const bool in = p / 16 < n;
        r[8 + u] = in ? *reinterpret_cast<const u32x4 *>(qu + (uint32_t)(p / 16) * rq + 8 * (p % 16))
                      : u32x4{0u, 0u, 0u, 0u};
        r[12 + u] = in ? *reinterpret_cast<const u32x4 *>(ku + (uint32_t)(p / 16) * rq + 8 * (p % 16))
                       : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // the v half: 8 pieces per row
        const int p = tid + NT * u;
        r[16 + u] = p / 8 < n ? __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                                    vu + (uint32_t)(p / 8) * rv + 8 * (p % 8)))
                              : u32x4{0u, 0u, 0u, 0u};
    }
    if (L > 0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            // the values read, made opaque to the compiler (a store of a value just loaded
            // from the same address would otherwise be dropped)
            const int p = tid + NT * u;
            u32x4 x = hr[u];
            asm volatile("" : "+v"(x));
            __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(hu + (uint32_t)(p / 16) * DV + 4 * (p % 16)));
        }
    }
    u32x4 acc = pacc;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= hr[u];
#pragma unroll
    for (int u = 0; u < 18; ++u) acc ^= r[u];
    float *ou = ly.out + (size_t)tr.lo * rv + (size_t)h * DV + c0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // the out half: 16 pieces per row
        const int p = tid + NT * u;
        if (p / 16 < n)
            __builtin_nontemporal_store(acc, reinterpret_cast<u32x4 *>(ou + (uint32_t)(p / 16) * rv + 4 * (p % 16)));
    }
}

bool aligned16(const void *a, const void *b, const void *c, const void *d, const void *e) {
    return ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
             reinterpret_cast<uintptr_t>(c) | reinterpret_cast<uintptr_t>(d) |
             reinterpret_cast<uintptr_t>(e)) & 15u) == 0;
}

}  // namespace

// Scalar-gate verify traffic. H0 [B, H, 128, 64] fp32, q and k [T, H, 128] bf16, v [T, H, 64]
// bf16, gate [T, H] fp32, out [T, H, 64] fp32 (written with arbitrary values),
// node_offsets [B + 1], all device pointers, 16-byte aligned. units_per_workgroup: 1, 2 or 4.
// Returns 0, -1 for a shape or alignment it does not take, or the launch's hipError_t.
PROBE_API int probe_verify_traffic_scalar(const float *H0, const void *q, const void *k,
                                          const void *v, const float *gate, float *out,
                                          const int32_t *node_offsets, int batch, int heads,
                                          int d_k, int d_v, int total_nodes,
                                          int units_per_workgroup, hipStream_t stream) {
    if (d_k != 128 || d_v != 64 || batch < 0 || heads <= 0 || total_nodes < 0) return -1;
    if (!aligned16(H0, q, k, v, out)) return -1;
    const int U = batch * heads;
    if (U == 0) return 0;
    const auto *qq = static_cast<const uint16_t *>(q);
    const auto *kk = static_cast<const uint16_t *>(k);
    const auto *vv = static_cast<const uint16_t *>(v);
    switch (units_per_workgroup) {
        case 1:
            scalar_traffic<1><<<U, 128, 0, stream>>>(H0, qq, kk, vv, gate, out, node_offsets, heads, U, total_nodes);
            break;
        case 2:
            scalar_traffic<2><<<(U + 1) / 2, 256, 0, stream>>>(H0, qq, kk, vv, gate, out, node_offsets, heads, U, total_nodes);
            break;
        case 4:
            scalar_traffic<4><<<(U + 3) / 4, 512, 0, stream>>>(H0, qq, kk, vv, gate, out, node_offsets, heads, U, total_nodes);
            break;
        default:
            return -1;
    }
    return (int)hipGetLastError();
}

// Vector-gate verify traffic: H0 [B, H, 128, 128] fp32, q and k [T, H, 128] bf16, v
// [T, H, 128] bf16, gate [T, H, 128] fp32, out [T, H, 128] fp32; otherwise as above.
PROBE_API int probe_verify_traffic_vector(const float *H0, const void *q, const void *k,
                                          const void *v, const float *gate, float *out,
                                          const int32_t *node_offsets, int batch, int heads,
                                          int d_k, int d_v, int total_nodes, hipStream_t stream) {
    if (d_k != 128 || d_v != 128 || batch < 0 || heads <= 0 || total_nodes < 0) return -1;
    if (!aligned16(H0, q, k, v, out) || (reinterpret_cast<uintptr_t>(gate) & 15u)) return -1;
    const int U = batch * heads;
    if (U == 0) return 0;
    vector_traffic<<<U, 512, 0, stream>>>(H0, static_cast<const uint16_t *>(q),
                                          static_cast<const uint16_t *>(k),
                                          static_cast<const uint16_t *>(v), gate, out,
                                          node_offsets, heads, total_nodes);
    return (int)hipGetLastError();
}

// Lazy-step traffic of nl <= 16 layers that share the trees and paths, one launch
// (blockIdx.y = layer): layers is a host array of nl ProbeLayer records (device pointers:
// H0 [B, H, 128, 64] fp32, read and written back unchanged; q, k [T, H, 128] and v
// [T, H, 64] bf16; gate [T, H] fp32; out [T, H, 64] fp32, written with arbitrary values;
// prev_k, prev_v, prev_gate the previous step's factors, [PT, H, ...]). node_offsets,
// prev_offsets [B + 1], accepted_idx [B, max_path], accepted_len [B] on the device. Paths
// of up to 64 nodes. Returns 0, -1 for a shape it does not take, or the hipError_t.
PROBE_API int probe_lazy_traffic_scalar(const ProbeLayer *layers, int nl,
                                        const int32_t *node_offsets, const int32_t *prev_offsets,
                                        const int32_t *accepted_idx, const int32_t *accepted_len,
                                        int batch, int heads, int d_k, int d_v, int total_nodes,
                                        int prev_total_nodes, int max_path, hipStream_t stream) {
    if (d_k != 128 || d_v != 64 || batch < 0 || heads <= 0 || nl < 1 || nl > kProbeLayers ||
        max_path < 1 || max_path > 64 || total_nodes < 0 || prev_total_nodes < 0)
        return -1;
    ProbeTable t = {};
    for (int l = 0; l < nl; ++l) {
        const ProbeLayer &y = layers[l];
        if (!aligned16(y.H0, y.q, y.k, y.v, y.out) || !aligned16(y.prev_k, y.prev_v, y.H0, y.H0, y.H0))
            return -1;
        t.l[l] = y;
    }
    const int U = batch * heads;
    if (U == 0) return 0;
    lazy_traffic<<<dim3((U + 1) / 2, nl), 256, 0, stream>>>(t, node_offsets, prev_offsets,
                                                            accepted_idx, accepted_len, max_path,
                                                            heads, U, total_nodes, prev_total_nodes);
    return (int)hipGetLastError();
}

// Lazy-step traffic with per-channel gates, nl <= 16 layers sharing the trees and paths, one
// launch: as probe_lazy_traffic_scalar with d_k = d_v = 128 and gate, prev_gate [T, H, 128]
// fp32 (H0 [B, H, 128, 128], q and k [T, H, 128], v [T, H, 128], out [T, H, 128]).
PROBE_API int probe_lazy_traffic_vector(const ProbeLayer *layers, int nl,
                                        const int32_t *node_offsets, const int32_t *prev_offsets,
                                        const int32_t *accepted_idx, const int32_t *accepted_len,
                                        int batch, int heads, int d_k, int d_v, int total_nodes,
                                        int prev_total_nodes, int max_path, hipStream_t stream) {
    if (d_k != 128 || d_v != 128 || batch < 0 || heads <= 0 || nl < 1 || nl > kProbeLayers ||
        max_path < 1 || max_path > 64 || total_nodes < 0 || prev_total_nodes < 0)
        return -1;
    ProbeTable t = {};
    for (int l = 0; l < nl; ++l) {
        const ProbeLayer &y = layers[l];
        if (!aligned16(y.H0, y.q, y.k, y.v, y.out) || !aligned16(y.prev_k, y.prev_v, y.gate, y.prev_gate, y.H0))
            return -1;
        t.l[l] = y;
    }
    const int U = batch * heads;
    if (U == 0) return 0;
    vector_lazy_traffic<<<dim3(((U + 7) / 8) * 16, nl), 256, 0, stream>>>(
        t, node_offsets, prev_offsets, accepted_idx, accepted_len, max_path, heads, U, total_nodes,
        prev_total_nodes);
    return (int)hipGetLastError();
}
