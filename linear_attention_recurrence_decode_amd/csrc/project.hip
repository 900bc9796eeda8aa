// project.hip -- fused input projections of the KDA layer on bf16 MFMA.
// [vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM", section
//  "KDA prefill and decode": the input projections are fused around the
//  recurrence.]
//
// One GEMM y = x W^T (x [T][Dm] bf16, W [N][Dm] bf16, fp32 accumulation)
// produces every per-token input of the layer; the epilogue routes each
// column to its tensor and applies the gate maps: q, k, v, z stored in the
// activation dtype, g = -softplus(y) and beta = sigmoid(y) in fp32.  The row
// blocks of W are q (H dk), k (H dk), v (H dv), z (H dv), g (H dk), beta (H).
//
// Tiling: 128 x 128 output tile per workgroup of 4 waves (2 x 2, each wave a
// 64 x 64 block of four 32x32x16 MFMA tiles), K in steps of 64 staged through
// two LDS buffers; the next step's tile is loaded into registers while the
// current one feeds the MFMAs.  Rows of x past T and of W past N read as zero
// through buffer resources.  Workgroups are mapped so that the tiles of one
// XCD (workgroups are dealt round-robin over the 8 XCDs) form 8-row groups
// sweeping N, so the concurrently running tiles of an XCD share panels of x
// and W in that XCD's L2.

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_p;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int BM = 128, BN = 128, BK = 64, LS = BK + 8;   // LDS row stride (bf16), padded
constexpr int NTH = 256;
constexpr int XCDS = 8, GROUP_M = 8;

union V16 {
    uint4 u;
    bf16x8_p v;
};

__device__ __forceinline__ float softplus_f(float y) {
    // max(y, 0) + log1p(exp(-|y|))
    return fmaxf(y, 0.f) + log1pf(__expf(-fabsf(y)));
}

__global__ __launch_bounds__(NTH) void project_kernel(ProjectParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LS];

    const int tiles_m = (p.T + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    // XCD-aware order: the workgroups an XCD receives get consecutive tile ids
    const int per_xcd = (tiles + XCDS - 1) / XCDS;
    const int b = blockIdx.x;
    const int tid_lin = (b % XCDS) * per_xcd + b / XCDS;
    if (tid_lin >= tiles) return;
    // grouped order: GROUP_M row tiles sweep all column tiles
    const int in_group = GROUP_M * tiles_n;
    const int gidx = tid_lin / in_group;
    const int first_m = gidx * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    const int tm = first_m + (tid_lin % in_group) % gm;
    const int tn = (tid_lin % in_group) / gm;
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int K = p.Dm;

    // tile loaders: 128 rows x 64 bf16 = 1024 16-byte units per operand, 4 per thread
    const auto ra = make_rsrc(static_cast<const uint16_t*>(p.x) + static_cast<int64_t>(m0) * K,
                              static_cast<uint32_t>(min(static_cast<int64_t>(BM), static_cast<int64_t>(p.T - m0)) * K * 2));
    const auto rb = make_rsrc(static_cast<const uint16_t*>(p.w) + static_cast<int64_t>(n0) * K,
                              static_cast<uint32_t>(min(static_cast<int64_t>(BN), static_cast<int64_t>(p.N - n0)) * K * 2));
    uint4 ga[4], gb[4];
    auto load = [&](int k0) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int u = tid + j * NTH, r = u >> 3, c = (u & 7) * 8;
            const uint32_t off = static_cast<uint32_t>((r * K + k0 + c) * 2);
            const float4 fa = buf_ld4(ra, off, 0), fb = buf_ld4(rb, off, 0);
            ga[j] = make_uint4(__float_as_uint(fa.x), __float_as_uint(fa.y), __float_as_uint(fa.z), __float_as_uint(fa.w));
            gb[j] = make_uint4(__float_as_uint(fb.x), __float_as_uint(fb.y), __float_as_uint(fb.z), __float_as_uint(fb.w));
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int u = tid + j * NTH, r = u >> 3, c = (u & 7) * 8;
            *reinterpret_cast<uint4*>(&As[buf][r * LS + c]) = ga[j];
            *reinterpret_cast<uint4*>(&Bs[buf][r * LS + c]) = gb[j];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;

    const int nk = K / BK;
    load(0);
    commit(0);
    __syncthreads();
    const int lr = lane & 31, lk = 8 * (lane >> 5);
    for (int ks = 0; ks < nk; ks++) {
        const int cur = ks & 1;
        if (ks + 1 < nk) load((ks + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            V16 a[2], bb[2];
#pragma unroll
            for (int i = 0; i < 2; i++)
                a[i].u = *reinterpret_cast<const uint4*>(&As[cur][(64 * wm + 32 * i + lr) * LS + kk + lk]);
#pragma unroll
            for (int j = 0; j < 2; j++)
                bb[j].u = *reinterpret_cast<const uint4*>(&Bs[cur][(64 * wn + 32 * j + lr) * LS + kk + lk]);
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i].v, bb[j].v, acc[i][j], 0, 0, 0);
        }
        if (ks + 1 < nk) commit(cur ^ 1);
        __syncthreads();
    }

    // epilogue: column n of y -> its tensor; element e of a 32x32 tile is at
    // row 8(e/4) + 4(lane/32) + e%4, column lane%32
    const int H = p.H, dk = p.dk, dv = p.dv;
    const int64_t bq = static_cast<int64_t>(H) * dk, bv = static_cast<int64_t>(H) * dv;
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int n = n0 + 64 * wn + 32 * j + lr;
        if (n >= p.N) continue;
        int kind;
        int64_t col, width;
        if (n < bq) { kind = 0; col = n; width = bq; }
        else if (n < 2 * bq) { kind = 1; col = n - bq; width = bq; }
        else if (n < 2 * bq + bv) { kind = 2; col = n - 2 * bq; width = bv; }
        else if (n < 2 * bq + 2 * bv) { kind = 3; col = n - 2 * bq - bv; width = bv; }
        else if (n < 3 * bq + 2 * bv) { kind = 4; col = n - 2 * bq - 2 * bv; width = bq; }
        else { kind = 5; col = n - 3 * bq - 2 * bv; width = H; }
        void* dst = kind == 0 ? p.q : kind == 1 ? p.k : kind == 2 ? p.v : kind == 3 ? p.z : kind == 4 ? p.g : p.beta;
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int m = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (m >= p.T) continue;
                const float y = acc[i][j][e];
                const int64_t o = static_cast<int64_t>(m) * width + col;
                if (kind < 4) static_cast<uint16_t*>(dst)[o] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(y));
                else if (kind == 4) static_cast<float*>(dst)[o] = -softplus_f(y);
                else static_cast<float*>(dst)[o] = sigmoid(y);
            }
    }
}

}  // namespace

hipError_t launch_project(const ProjectParams& p, hipStream_t s) {
    const int64_t tiles = static_cast<int64_t>((p.T + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    if (tiles == 0) return hipSuccess;
    const int64_t grid = (tiles + XCDS - 1) / XCDS * XCDS;
    hipLaunchKernelGGL(project_kernel, dim3(static_cast<unsigned>(grid)), dim3(NTH), 0, s, p);
    return hipGetLastError();
}

}  // namespace kda
