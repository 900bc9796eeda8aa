// project.hip -- input and output projections of the KDA layer on bf16 MFMA.
// [vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM", section
//  "KDA prefill and decode": the input projections are fused around the
//  recurrence.]
//
// One GEMM y = x W^T (x [T][Dm] bf16, W [N][Dm] bf16, fp32 accumulation)
// produces every per-token input of the layer; the epilogue routes each
// column to its tensor and applies the gate maps: q, k, v, z stored in the
// activation dtype, g = -softplus(y) and beta = sigmoid(y) in fp32.  The row
// blocks of W are q (H dk), k (H dk), v (H dv), z (H dv), g (H dk), beta (H).
// The same kernel in its second mode is the output projection: the layer's
// output o [T][H dv] times W_o [Dm][H dv]^T, stored as bf16 [T][Dm].
//
// Tiling: a 256 x 256 output tile per workgroup of 8 waves (2 x 4, each wave
// a 128 x 64 block of eight 32x32x16 MFMA tiles, two waves per SIMD), K in
// steps of 64.  The x and W tiles of a step are copied from global memory
// straight into LDS (buffer loads with the LDS destination bit, no register
// staging) into one of two buffers while the other feeds the MFMAs; the LDS
// rows are unpadded with an XOR swizzle of their 16-byte chunks, so that both
// the copies (1 KiB contiguous per wave instruction) and the fragment reads
// are free of bank conflicts.  Workgroups are mapped so that the tiles of one
// XCD form groups of 4 row tiles sweeping N, sharing panels of x and W in
// that XCD's L2.  The epilogue stages the fp32 results through LDS.

#include <utility>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_p;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int XCDS = 8, GROUP_M = 4;

union V16 {
    uint4 u;
    bf16x8_p v;
};

// softplus(y) = max(y, 0) + log1p(e), e = exp(-|y|) in (0, 1].  log1p(e) is
// taken as 2 atanh(s) with s = e / (2 + e) in (0, 1/3]: the odd series
// 2 s (1 + s^2/3 + s^4/5 + ... + s^14/15), whose first omitted term is below
// 2^-28 of the sum.  One reciprocal and eight FMAs, about a third of the
// instructions of a library log1pf, for a few ulp.  y = -inf gives 0, +inf
// gives +inf, NaN stays NaN.
__device__ __forceinline__ float softplus_f(float y) {
    const float e = __expf(-fabsf(y));
    const float s = e * __builtin_amdgcn_rcpf(2.0f + e);
    const float s2 = s * s;
    float p = 1.0f / 15.0f;
    p = fmaf(p, s2, 1.0f / 13.0f);
    p = fmaf(p, s2, 1.0f / 11.0f);
    p = fmaf(p, s2, 1.0f / 9.0f);
    p = fmaf(p, s2, 1.0f / 7.0f);
    p = fmaf(p, s2, 1.0f / 5.0f);
    p = fmaf(p, s2, 1.0f / 3.0f);
    p = fmaf(p, s2, 1.0f);
    return fmaxf(y, 0.f) + 2.0f * s * p;
}

// Output tile of this workgroup, or false past the last tile.  Workgroups are
// dealt round-robin over the 8 XCDs, so the ids an XCD receives are made
// consecutive; within an XCD, groups of GROUP_M row tiles sweep all column
// tiles so that the concurrently running tiles share panels of x and W in
// that XCD's L2.
// Rows of the causal conv's window before the current token.
constexpr int HALO = 3;

template <int BM, int BN>
__device__ __forceinline__ bool tile_origin(const ProjectParams& p, int& m0, int& n0) {
    const int tiles_m = (p.T + BM - 1) / BM, tiles_n = (p.N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int per_xcd = (tiles + XCDS - 1) / XCDS;
    const int b = blockIdx.x;
    const int t = (b % XCDS) * per_xcd + b / XCDS;
    if (t >= tiles) return false;
    const int in_group = GROUP_M * tiles_n;
    const int first_m = (t / in_group) * GROUP_M;
    const int gm = min(tiles_m - first_m, GROUP_M);
    m0 = (first_m + (t % in_group) % gm) * BM;
    n0 = ((t % in_group) / gm) * BN;
    return true;
}

// Epilogue, one 32-row strip of the wave's block at a time: the fp32 tiles go
// through LDS (element e of a 32x32 tile is at row 8(e/4) + 4(lane/32) + e%4,
// column lane%32) and come back as 4 consecutive columns of one row per lane,
// so that a group's routing (tensor, offset, gate map) is worked out once and
// its 4 results leave in one 8-byte (bf16) or 16-byte (fp32) store.  The
// tensor blocks of the input projections start at multiples of 32 columns, so
// a group never straddles two tensors; a group that runs past N, a row width
// that is not a multiple of 4 or a destination that is not aligned for the
// wide store is written element by element.  The tile buffers must be free
// (all waves past their last read) on entry.
template <int BM, int BN, int WM, int WN, int TI = BM / WM / 32, int TJ = BN / WN / 32>
__device__ __forceinline__ void epilogue(const ProjectParams& p, const f32x16 (&acc)[TI][TJ], float* smem, int m0,
                                         int n0) {
    constexpr int RM = BM / WM, RN = BN / WN;
    constexpr int EP = RN + 4;              // staging row stride (floats)
    constexpr int GPR = RN / 4;             // 4-column groups per row
    constexpr int RPI = 64 / GPR;           // rows per store instruction
    static_assert(RN % 4 == 0 && 64 % GPR == 0 && 32 % RPI == 0, "column groups must tile a wave");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lr = lane & 31;
    const int wm = wave / WN, wn = wave % WN;
    float* stage = smem + wave * 32 * EP;
    const int cg = lane % GPR, rsub = lane / GPR;

    // routing of this lane's 4 columns n .. n+3
    const int H = p.H, dk = p.dk, dv = p.dv;
    const int64_t bq = static_cast<int64_t>(H) * dk, bv = static_cast<int64_t>(H) * dv;
    const int64_t n = n0 + RN * wn + 4 * cg;
    const int nv = static_cast<int>(min(static_cast<int64_t>(4), max(static_cast<int64_t>(0), p.N - n)));
    int kind;
    int64_t col, width;
    if (nv == 0) { kind = -1; col = 0; width = 0; }
    else if (p.mode == 1) { kind = 0; col = n; width = p.N; }
    else if (n < bq) { kind = 0; col = n; width = bq; }
    else if (n < 2 * bq) { kind = 1; col = n - bq; width = bq; }
    else if (n < 2 * bq + bv) { kind = 2; col = n - 2 * bq; width = bv; }
    else if (n < 2 * bq + 2 * bv) { kind = 3; col = n - 2 * bq - bv; width = bv; }
    else if (n < 3 * bq + 2 * bv) { kind = 4; col = n - 2 * bq - 2 * bv; width = bq; }
    else { kind = 5; col = n - 3 * bq - 2 * bv; width = H; }
    void* dst = p.mode == 1 ? p.y : kind == 0 ? p.q : kind == 1 ? p.k : kind == 2 ? p.v : kind == 3 ? p.z
                                  : kind == 4 ? p.g : p.beta;
    const int esz = kind >= 4 ? 4 : 2;
    const bool wide = nv == 4 && width % 4 == 0 && col % 4 == 0 && reinterpret_cast<uintptr_t>(dst) % (4 * esz) == 0;

#pragma unroll
    for (int i = 0; i < TI; i++) {
#pragma unroll
        for (int j = 0; j < TJ; j++)
#pragma unroll
            for (int e = 0; e < 16; e++)
                stage[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * EP + 32 * j + lr] = acc[i][j][e];
        __syncthreads();
        const int mb = m0 + RM * wm + 32 * i;
#pragma unroll 2
        for (int it = 0; it < 32 / RPI; it++) {
            const int r = it * RPI + rsub;
            const int m = mb + r;
            if (kind < 0 || m >= p.T) continue;
            const float4 y = *reinterpret_cast<const float4*>(&stage[r * EP + 4 * cg]);
            const int64_t o = static_cast<int64_t>(m) * width + col;
            float v4[4] = {y.x, y.y, y.z, y.w};
            if (kind == 4) {
#pragma unroll
                for (int c = 0; c < 4; c++) v4[c] = -softplus_f(v4[c]);
            } else if (kind == 5) {
#pragma unroll
                for (int c = 0; c < 4; c++) v4[c] = sigmoid(v4[c]);
            }
            if (wide) {
                if (kind < 4) {
                    uint2 w;
                    w.x = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v4[0]))) |
                          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v4[1]))) << 16);
                    w.y = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v4[2]))) |
                          (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v4[3]))) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + o) = w;
                } else {
                    *reinterpret_cast<float4*>(static_cast<float*>(dst) + o) = make_float4(v4[0], v4[1], v4[2], v4[3]);
                }
            } else {
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    if (c >= nv) break;
                    if (kind < 4) static_cast<uint16_t*>(dst)[o + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v4[c]));
                    else static_cast<float*>(dst)[o + c] = v4[c];
                }
            }
        }
        __syncthreads();
    }
}

// SiLU of the conv front end: exp through the hardware base-2 exponential
// and the hardware reciprocal (a few ulp in fp32, far below the bf16 rounding
// of the result).  y -> -inf gives exp2 -> inf, rcp -> 0 and -0; no NaN.
__device__ __forceinline__ float front_silu(float y) {
    return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * y));
}

// Post-conv activation of one channel from its window of rounded raw inputs
// (oldest first); the epilogue and the tile-top pass use this one expression,
// so that a row gets the same bits whichever computes it.
__device__ __forceinline__ float front_act(const float4& w, float a, float b, float c, float d) {
    return front_silu(conv4(w, a, b, c, d));
}

template <int... I, typename F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F&& f) {
    (f(std::integral_constant<int, I>{}), ...);
}

__device__ __forceinline__ float round_bf16(float x) { return static_cast<float>(static_cast<__bf16>(x)); }

// Sequence of packed row m (0 <= m < cu[num_seqs]): the largest n with
// cu[n] <= m, which skips empty sequences.  Returns (cu[n], n).
__device__ __forceinline__ int2 sequence_of(const int32_t* cu, int num_seqs, int m) {
    int lo = 0, hi = num_seqs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= m) lo = mid;
        else hi = mid;
    }
    return make_int2(cu[lo], lo);
}

// Left-context value of conv channel ch of head `head` for the row `back`
// rows before a sequence's first token (back = 1 .. 3): the sequence's
// initial conv state (index 3 - back; 2 = the token just before the start)
// or zero without one.
__device__ __forceinline__ float conv_context(const ProjectParams& p, int seq, int head, int ch, int back) {
    const int slot = (p.init_slot && seq >= 0) ? p.init_slot[seq] : -1;
    if (slot < 0 || slot >= p.num_slots) return 0.f;
    const int C = 2 * p.dk + p.dv;
    return bf16_to_f32(static_cast<const uint16_t*>(p.conv_pool)[
        ((static_cast<int64_t>(slot) * p.H + head) * C + ch) * HALO + (HALO - back)]);
}

// Store of 4 consecutive results of one row: one 8-byte (bf16) or 16-byte
// (fp32) store when `wide`, else element by element.
__device__ __forceinline__ void put4(void* base, int64_t o, bool wide, bool is_f32, int nv, const float (&x)[4]) {
    if (wide) {
        if (!is_f32) {
            uint2 w;
            w.x = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x[0]))) |
                  (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x[1]))) << 16);
            w.y = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x[2]))) |
                  (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(x[3]))) << 16);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + o) = w;
        } else {
            *reinterpret_cast<float4*>(static_cast<float*>(base) + o) = make_float4(x[0], x[1], x[2], x[3]);
        }
    } else {
#pragma unroll
        for (int c = 0; c < 4; c++) {
            if (c >= nv) break;
            if (!is_f32) static_cast<uint16_t*>(base)[o + c] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x[c]));
            else static_cast<float*>(base)[o + c] = x[c];
        }
    }
}

// Epilogue of the conv front end.  The routing is that of `epilogue`; on the
// q, k and v columns each row m becomes
//   raw(m)  = RNE_bf16(x W^T)                       (stored in the second tensor)
//   a(m)    = RNE_bf16(SiLU(conv4(w, raw(m-3), raw(m-2), raw(m-1), raw(m))))
// where a row before its sequence's first token is taken from that
// sequence's initial conv state (index 2 = the token just before the start)
// or is zero, exactly as the prefill forms its left context; z, g and beta
// are stored as in `epilogue`.
// Each lane owns 4 columns of RPS consecutive rows of a 32-row strip and
// slides the window down them: a row is read from LDS and rounded once, and
// its three predecessors stay in registers.  A lane whose rows and window lie
// in one sequence past its first HALO tokens takes no boundary test.  The
// rows before a strip come from the previous strip (kept in `halo`), for the
// second row-wave's first strip from the first row-wave's last strip; the
// tile's first HALO rows, whose window reaches into the previous tile, get
// their activations from conv_tile_top_kernel after the GEMM (their raw
// inputs are stored here).
template <int BM, int BN, int WM, int WN, int TI = BM / WM / 32, int TJ = BN / WN / 32>
__device__ __forceinline__ void epilogue_conv(const ProjectParams& p, const f32x16 (&acc)[TI][TJ], float* smem,
                                              int m0, int n0) {
    constexpr int RM = BM / WM, RN = BN / WN, NW = WM * WN;
    constexpr int EP = RN + 4;
    constexpr int GPR = RN / 4;             // 4-column groups per row
    constexpr int SEGS = 64 / GPR;          // row segments per strip
    constexpr int RPS = 32 / SEGS;          // rows per segment
    static_assert(RN % 4 == 0 && GPR * SEGS == 64 && RPS * SEGS == 32 && RPS >= HALO,
                  "column groups and row segments must tile a wave's strip");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, lr = lane & 31;
    const int wm = wave / WN, wn = wave % WN;
    float* stage = smem + wave * 32 * EP;
    float* halo_all = smem + NW * 32 * EP;                                 // [NW][HALO][EP]
    float* halo = halo_all + wave * HALO * EP;
    int2* rowinfo = reinterpret_cast<int2*>(halo_all + NW * HALO * EP);   // [BM]: (sequence start, sequence)
    const int cg = lane % GPR, seg = lane / GPR;

    const int H = p.H, dk = p.dk, dv = p.dv, C = 2 * dk + dv;
    const int64_t bq = static_cast<int64_t>(H) * dk, bv = static_cast<int64_t>(H) * dv;
    const int64_t n = n0 + RN * wn + 4 * cg;
    const int nv = static_cast<int>(min(static_cast<int64_t>(4), max(static_cast<int64_t>(0), p.N - n)));
    int kind;
    int64_t col, width;
    if (nv == 0) { kind = -1; col = 0; width = 0; }
    else if (n < bq) { kind = 0; col = n; width = bq; }
    else if (n < 2 * bq) { kind = 1; col = n - bq; width = bq; }
    else if (n < 2 * bq + bv) { kind = 2; col = n - 2 * bq; width = bv; }
    else if (n < 2 * bq + 2 * bv) { kind = 3; col = n - 2 * bq - bv; width = bv; }
    else if (n < 3 * bq + 2 * bv) { kind = 4; col = n - 2 * bq - 2 * bv; width = bq; }
    else { kind = 5; col = n - 3 * bq - 2 * bv; width = H; }
    void* dst = kind == 0 ? p.q : kind == 1 ? p.k : kind == 2 ? p.v : kind == 3 ? p.z : kind == 4 ? p.g : p.beta;
    const bool is_f32 = kind >= 4;
    const bool wide = nv == 4 && width % 4 == 0 && col % 4 == 0 &&
                      reinterpret_cast<uintptr_t>(dst) % (is_f32 ? 16 : 8) == 0;
    // conv channel and weights of this lane's columns (q, k, v only; the 4
    // columns of a group lie in one head: the head sizes are multiples of 32)
    const bool convk = kind >= 0 && kind <= 2;
    const int dh = kind == 2 ? dv : dk;
    const int head = convk ? static_cast<int>(col / dh) : 0;
    const int cc = convk ? kind * dk + static_cast<int>(col % dh) : 0;   // first conv channel of the group
    float4 cw[4];
#pragma unroll
    for (int c = 0; c < 4; c++)
        cw[c] = (convk && c < nv) ? *reinterpret_cast<const float4*>(p.conv_w + (static_cast<int64_t>(head) * C + cc + c) * 4)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
    void* raw_dst = convk ? static_cast<void*>(static_cast<uint16_t*>(dst) + static_cast<int64_t>(p.T) * width) : dst;

    // sequence start and index of every tile row; rows past T get a start no
    // row reaches, which keeps their lanes off the fast path
    for (int r = threadIdx.x; r < BM; r += 64 * NW) {
        const int m = m0 + r;
        rowinfo[r] = m < p.T ? sequence_of(p.cu_seqlens, p.num_seqs, m) : make_int2(INT32_MAX, -1);
    }

    // Strips by compile-time index, so that acc stays in registers; the row
    // loops inside stay rolled (the epilogue runs once per tile, and fully
    // unrolled its code would be fetched cold line after line).
    static_for(std::make_integer_sequence<int, TI>{}, [&](auto strip) {
        constexpr int i = decltype(strip)::value;
#pragma unroll
        for (int j = 0; j < TJ; j++)
#pragma unroll
            for (int e = 0; e < 16; e++)
                stage[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * EP + 32 * j + lr] = acc[i][j][e];
        if (i == 0 && WM > 1 && wm == 0 && lane >= 32) {
            // rows RM-3 .. RM-1 (the last strip's rows 29..31: e = 13..15 of
            // the upper half-wave) are the left context of the next row-wave
            float* dh2 = halo_all + (wave + WN) * HALO * EP;
#pragma unroll
            for (int j = 0; j < TJ; j++)
#pragma unroll
                for (int e = 13; e < 16; e++) dh2[((e & 3) - 1) * EP + 32 * j + lr] = acc[TI - 1][j][e];
        }
        __syncthreads();
        const int r0 = RPS * seg;                       // this lane's first strip row
        const int tr0 = RM * wm + 32 * i + r0;          // ... as a tile row
        const int mr0 = m0 + tr0;
        int64_t o = static_cast<int64_t>(mr0) * width + col;
        if (kind >= 0 && mr0 < p.T) {
            if (convk) {
                float w3[4], w2[4], w1[4];              // rounded raw rows r-3, r-2, r-1
                auto load = [&](int r, float (&x)[4]) {
                    const float4 y = *reinterpret_cast<const float4*>(
                        r >= 0 ? &stage[r * EP + 4 * cg] : &halo[(r + HALO) * EP + 4 * cg]);
                    x[0] = round_bf16(y.x);
                    x[1] = round_bf16(y.y);
                    x[2] = round_bf16(y.z);
                    x[3] = round_bf16(y.w);
                };
                load(r0 - 3, w3);
                load(r0 - 2, w2);
                load(r0 - 1, w1);
                const bool fast = rowinfo[tr0 + RPS - 1].x <= mr0 - HALO;
#pragma unroll 1
                for (int t = 0; t < RPS; t++) {
                    const int m = mr0 + t;
                    float w0[4];
                    load(r0 + t, w0);
                    float b3[4], b2[4], b1[4];
#pragma unroll
                    for (int c = 0; c < 4; c++) { b3[c] = w3[c]; b2[c] = w2[c]; b1[c] = w1[c]; }
                    if (!fast && m < p.T) {
                        // rows before the sequence's first token: its initial conv state or zero
                        // (si.x <= m, so the context index si.x - (m - j) is 1 .. j)
                        const int2 si = rowinfo[tr0 + t];
                        if (m - 3 < si.x) {
#pragma unroll
                            for (int c = 0; c < 4; c++) {
                                if (c >= nv) break;
                                if (m - 1 < si.x) b1[c] = conv_context(p, si.y, head, cc + c, si.x - (m - 1));
                                if (m - 2 < si.x) b2[c] = conv_context(p, si.y, head, cc + c, si.x - (m - 2));
                                b3[c] = conv_context(p, si.y, head, cc + c, si.x - (m - 3));
                            }
                        }
                    }
                    if (m < p.T) {
                        if (tr0 + t >= HALO) {
                            float a4[4];
#pragma unroll
                            for (int c = 0; c < 4; c++) a4[c] = front_act(cw[c], b3[c], b2[c], b1[c], w0[c]);
                            put4(dst, o, wide, false, nv, a4);
                        }
                        put4(raw_dst, o, wide, false, nv, w0);
                    }
#pragma unroll
                    for (int c = 0; c < 4; c++) { w3[c] = w2[c]; w2[c] = w1[c]; w1[c] = w0[c]; }
                    o += width;
                }
            } else {
#pragma unroll 1
                for (int t = 0; t < RPS; t++) {
                    if (mr0 + t < p.T) {
                        const float4 y = *reinterpret_cast<const float4*>(&stage[(r0 + t) * EP + 4 * cg]);
                        float v4[4] = {y.x, y.y, y.z, y.w};
                        if (kind == 4) {
#pragma unroll
                            for (int c = 0; c < 4; c++) v4[c] = -softplus_f(v4[c]);
                        } else if (kind == 5) {
#pragma unroll
                            for (int c = 0; c < 4; c++) v4[c] = sigmoid(v4[c]);
                        }
                        put4(dst, o + t * width, wide, is_f32, nv, v4);
                    }
                }
            }
        }
        // this strip's last HALO rows are the next strip's left context
        if (i + 1 < TI) {
            for (int e = lane; e < HALO * RN; e += 64) {
                const int hr = e / RN, hc = e % RN;
                halo[hr * EP + hc] = stage[(32 - HALO + hr) * EP + hc];
            }
        }
        __syncthreads();
    });
}

// Activations of the first HALO rows of every BM-row tile of the conv front
// end, whose window reaches into the tile above: one channel of one row per
// thread, from the raw inputs the GEMM stored (the same rounded values its
// epilogue holds) and, before a sequence's first token, its initial conv state.
__global__ __launch_bounds__(256) void conv_tile_top_kernel(ProjectParams p, int BM) {
    const int H = p.H, dk = p.dk, dv = p.dv, C = 2 * dk + dv;
    const int64_t bq = static_cast<int64_t>(H) * dk, bv = static_cast<int64_t>(H) * dv;
    const int64_t ncol = 2 * bq + bv;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t row = e / ncol, n = e % ncol;           // row: (tile, HALO row of the tile)
    const int m = static_cast<int>(row / HALO) * BM + static_cast<int>(row % HALO);
    if (m >= p.T) return;
    int kind;
    int64_t col, width;
    if (n < bq) { kind = 0; col = n; width = bq; }
    else if (n < 2 * bq) { kind = 1; col = n - bq; width = bq; }
    else { kind = 2; col = n - 2 * bq; width = bv; }
    uint16_t* dst = static_cast<uint16_t*>(kind == 0 ? p.q : kind == 1 ? p.k : p.v);
    const uint16_t* raw = dst + static_cast<int64_t>(p.T) * width;
    const int dh = kind == 2 ? dv : dk;
    const int head = static_cast<int>(col / dh), ch = kind * dk + static_cast<int>(col % dh);
    const int2 si = sequence_of(p.cu_seqlens, p.num_seqs, m);
    float x[HALO + 1];                                    // rows m-3 .. m
#pragma unroll
    for (int j = 0; j <= HALO; j++) {
        const int mj = m - HALO + j;
        x[j] = mj >= si.x ? bf16_to_f32(raw[static_cast<int64_t>(mj) * width + col])
                          : conv_context(p, si.y, head, ch, si.x - mj);
    }
    const float4 w = *reinterpret_cast<const float4*>(p.conv_w + (static_cast<int64_t>(head) * C + ch) * 4);
    dst[static_cast<int64_t>(m) * width + col] =
        __builtin_bit_cast(uint16_t, static_cast<__bf16>(front_act(w, x[0], x[1], x[2], x[3])));
}

// Physical 16-byte chunk of logical chunk c in row r of an unpadded LDS tile
// with CPR chunks per row (XOR is its own inverse, so the same map takes a
// physical chunk to its logical one).  For every aligned run of 8 rows, and
// of 16 rows taken with the row's position in a 256-byte bank period, the
// chunks read by one fragment load land in distinct banks.
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
    if constexpr (CPR == 8) return c ^ ((r ^ (r >> 3)) & 7);
    else return c ^ (((r >> 1) ^ (r >> 3)) & 3);
}

// One wave copy of 1 KiB into LDS at byte address `lds` (uniform): lane L
// loads 16 bytes at voff + soff of the buffer and writes them at lds + 16 L.
// Issued as inline assembly, so that the compiler, which cannot tell which
// LDS bytes such a copy writes, does not wait for the copies in flight before
// every LDS read; the kernel waits for its copies itself, at the barriers.
__device__ __forceinline__ void copy_to_lds(i32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory", "m0");
}

// Wait until this wave's copies have landed and its LDS reads have returned,
// then a workgroup barrier: one unit that the compiler neither splits nor
// moves memory accesses across.
__device__ __forceinline__ void wait_copies_and_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

__device__ __forceinline__ i32x4 raw_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    i32x4 r;
    r[0] = static_cast<int32_t>(a);
    r[1] = static_cast<int32_t>((a >> 32) & 0xffff);
    r[2] = static_cast<int32_t>(bytes);
    r[3] = 0x00020000;
    return r;
}

// BM x BN output tile per workgroup of WM x WN waves, each wave a (BM/WM) x
// (BN/WN) block of TI x TJ tiles of 32x32, K in steps of BK.  The global tiles
// are copied straight into LDS (buffer_load ... lds, 16 bytes per lane: a wave
// instruction fills 1 KiB of LDS contiguously), one step ahead, into two
// buffers; no registers hold them.  Rows past T (or N) read the last valid
// row instead; they only feed outputs that are never stored.
template <int BM, int BN, int BK, int WM, int WN, bool CONV>
__global__ __launch_bounds__(64 * WM * WN) void project_kernel(ProjectParams p) {
    constexpr int NW = WM * WN;
    constexpr int RM = BM / WM, RN = BN / WN;
    constexpr int TI = RM / 32, TJ = RN / 32;
    constexpr int RB = 2 * BK, CPR = BK / 8;      // bytes and 16-byte chunks per row
    constexpr int RPI = 1024 / RB;                // rows per wave copy instruction
    constexpr int IA = BM / (RPI * NW), IB = BN / (RPI * NW);
    static_assert(IA * RPI * NW == BM && IB * RPI * NW == BN, "tile rows must split evenly over the waves");
    constexpr int SA = BM * RB, SS = (BM + BN) * RB;   // bytes: A part of a buffer, whole buffer
    constexpr int KK = BK / 16;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * SS];

    int m0, n0;
    if (!tile_origin<BM, BN>(p, m0, n0)) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int K = p.Dm;
    const int va_rows = min(BM, p.T - m0), vb_rows = min(BN, p.N - n0);
    const i32x4 ra = raw_rsrc(static_cast<const uint16_t*>(p.x) + static_cast<int64_t>(m0) * K,
                              static_cast<uint32_t>(va_rows) * K * 2);
    const i32x4 rb = raw_rsrc(static_cast<const uint16_t*>(p.w) + static_cast<int64_t>(n0) * K,
                              static_cast<uint32_t>(vb_rows) * K * 2);
    // per-lane global offsets (the step's k offset goes in soffset)
    uint32_t oa[IA], ob[IB];
#pragma unroll
    for (int j = 0; j < IA; j++) {
        const int r = (wave * IA + j) * RPI + lane / CPR;
        oa[j] = static_cast<uint32_t>((min(r, va_rows - 1) * K + 8 * swz<CPR>(r, lane % CPR)) * 2);
    }
#pragma unroll
    for (int j = 0; j < IB; j++) {
        const int r = (wave * IB + j) * RPI + lane / CPR;
        ob[j] = static_cast<uint32_t>((min(r, vb_rows - 1) * K + 8 * swz<CPR>(r, lane % CPR)) * 2);
    }
    const uint32_t lds0 = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(smem)));
    const int nk = K / BK;
    auto issue = [&](int step) {
        if (step >= nk) return;
        const uint32_t st = __builtin_amdgcn_readfirstlane(lds0 + (step & 1) * SS + wave * (IA * 1024));
        const uint32_t stb = __builtin_amdgcn_readfirstlane(lds0 + (step & 1) * SS + SA + wave * (IB * 1024));
        const uint32_t soff = __builtin_amdgcn_readfirstlane(step * BK * 2);
#pragma unroll
        for (int j = 0; j < IA; j++) copy_to_lds(ra, st + j * 1024, oa[j], soff);
#pragma unroll
        for (int j = 0; j < IB; j++) copy_to_lds(rb, stb + j * 1024, ob[j], soff);
    };

    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; i++)
#pragma unroll
        for (int j = 0; j < TJ; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.f;

    const int lr = lane & 31, hi = lane >> 5;
    V16 fa[2][TI], fb[2][TJ];
    auto frags = [&](int slot, const uint8_t* st, int q) {
#pragma unroll
        for (int i = 0; i < TI; i++) {
            const int r = RM * wm + 32 * i + lr;
            fa[slot][i].u = *reinterpret_cast<const uint4*>(st + r * RB + 16 * swz<CPR>(r, 2 * q + hi));
        }
#pragma unroll
        for (int j = 0; j < TJ; j++) {
            const int r = RN * wn + 32 * j + lr;
            fb[slot][j].u = *reinterpret_cast<const uint4*>(st + SA + r * RB + 16 * swz<CPR>(r, 2 * q + hi));
        }
    };
    auto mma = [&](int slot) {
#pragma unroll
        for (int i = 0; i < TI; i++)
#pragma unroll
            for (int j = 0; j < TJ; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][i].v, fb[slot][j].v, acc[i][j], 0, 0, 0);
    };

    // Two buffers: the copy of step ks + 2 may only start once every wave has
    // read its last fragments of step ks (same buffer), and step ks + 1 must
    // have landed before its first fragments are read.  One barrier after the
    // last fragment read of each step serves both; the MFMAs of that step's
    // last sub-step, whose operands are already in registers, then cover the
    // burst of first-fragment reads of step ks + 1 that follows the barrier.
    issue(0);
    wait_copies_and_barrier();
    issue(1);
    frags(0, smem, 0);
    for (int ks = 0; ks < nk; ks++) {
        const uint8_t* st = smem + (ks & 1) * SS;
#pragma unroll
        for (int q = 0; q + 1 < KK; q++) {
            frags((q + 1) & 1, st, q + 1);
            mma(q & 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 1 < nk) {
            wait_copies_and_barrier();
            __builtin_amdgcn_sched_barrier(0);
            frags(KK & 1, smem + ((ks + 1) & 1) * SS, 0);
            __builtin_amdgcn_sched_barrier(0);
            issue(ks + 2);
        }
        mma((KK - 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    static_assert(NW * 32 * (RN + 4) * 4 <= sizeof(smem), "epilogue staging exceeds the tile buffers");
    static_assert(NW * (32 + HALO) * (RN + 4) * 4 + BM * 8 <= sizeof(smem), "conv staging exceeds the tile buffers");
    if constexpr (CONV) epilogue_conv<BM, BN, WM, WN>(p, acc, reinterpret_cast<float*>(smem), m0, n0);
    else epilogue<BM, BN, WM, WN>(p, acc, reinterpret_cast<float*>(smem), m0, n0);
}

}  // namespace

hipError_t launch_project(const ProjectParams& p, hipStream_t s) {
    constexpr int BM = 256, BN = 256, BK = 64, WM = 2, WN = 4;
    const int64_t tiles_m = (p.T + BM - 1) / BM;
    const int64_t tiles = tiles_m * ((p.N + BN - 1) / BN);
    if (tiles == 0) return hipSuccess;
    const int64_t grid = (tiles + XCDS - 1) / XCDS * XCDS;
    // tile ids and the per-lane byte offsets ((row < BM) x Dm + chunk) x 2 are 32-bit
    if (grid > INT32_MAX || (static_cast<int64_t>(BM - 1) * p.Dm + BK) * 2 > INT32_MAX) return hipErrorInvalidValue;
    if (p.conv) {
        hipLaunchKernelGGL((project_kernel<BM, BN, BK, WM, WN, true>), dim3(static_cast<unsigned>(grid)),
                           dim3(64 * WM * WN), 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int64_t items = tiles_m * HALO * (static_cast<int64_t>(p.H) * (2 * p.dk + p.dv));
        const int64_t blocks = (items + 255) / 256;
        if (blocks > INT32_MAX) return hipErrorInvalidValue;
        hipLaunchKernelGGL(conv_tile_top_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, BM);
    } else {
        hipLaunchKernelGGL((project_kernel<BM, BN, BK, WM, WN, false>), dim3(static_cast<unsigned>(grid)),
                           dim3(64 * WM * WN), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace kda
