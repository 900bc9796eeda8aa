// prefill.hip -- chunked KDA prefill over packed variable-length sequences
// for gfx950, with recurrent-state checkpoints.
//
// [vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM",
//  section "KDA prefill and decode": the prefill gathers each request's
//  initial recurrent state in one operation and runs a chunked kernel around
//  the recurrence; section "The Hardest Part: Prefix Caching for KDA": a
//  resumable state must exist at exact prefix boundaries; agentlenshq "vLLM
//  Kimi K3 Support", section "Agentic Cache Retention Policies": states are
//  kept at fixed intervals and at prompt ends.]
//
// Chunked form.  For a chunk of n <= 64 tokens entered with state S
// (dk x dv), Gam the within-chunk cumulative log-decay per key channel, and
// the gated delta rule S_t = (I - b_t k_t k_t^T) Diag(exp g_t) S_{t-1} +
// b_t k_t v_t^T unrolled over the chunk:
//   M[t,s] = sum_i k[t,i] k[s,i] exp(Gam[t,i] - Gam[s,i])   (s <  t)
//   P[t,s] = sum_i q[t,i] k[s,i] exp(Gam[t,i] - Gam[s,i])   (s <= t)
//   T      = (I + Diag(b) M)^{-1}                              (unit lower)
//   U      = T Diag(b) (V - (k * exp(Gam)) S)                  (the chunk's u_t)
//   O      = (q * exp(Gam)) S + P U                            (readouts)
//   S'     = Diag(exp Gam_end) S + (k * exp(Gam_end - Gam))^T U
// The pairwise decays are factored through a reference row r = 31 (the
// chunk's middle): k*exp(Gam - Gam_r) times k*exp(Gam_r - Gam).  Per-channel
// factors exp(Gam_r), exp(Gam_end - Gam_r) and exp(Gam_end) then move onto the
// state side, so the three stored operands K+ = k exp(Gam-Gam_r),
// K- = k exp(Gam_r-Gam), Q+ = q exp(Gam-Gam_r) serve every product.  This needs
// |Gam_t - Gam_r| inside the fp32 exponent range for every channel; a chunk
// with a channel whose decay over one of its 16-row blocks reaches -40 (or a
// gate of -inf) takes a block-local form instead, with every factor <= 1
// (local_planes, local_products, local_rescale), so any g <= 0 is handled.
//
// Workgroup = one (sequence, head) chain, NW = dv/16 waves, chunks in order.
// Phase A (state independent): raw rows staged in LDS, causal conv + SiLU,
// L2 norms, cumulative decay, K+/K-/Q+ as bf16 hi/lo planes, L = Diag(b) M
// and P on MFMA, and the inverses of the four 16x16 diagonal blocks of I + L
// by forward substitution in fp32 (eight threads per column).  T itself is
// never formed: phase B solves (I + L) U = Y block by block,
// U_a = T_aa (Y_a - sum_{c<a} L_ac U_c).
// Phase B (state dependent): wave w owns columns [16w, 16w+16) of S in MFMA
// accumulator layout (lane l: rows 4(l/16)+e of each 16-row tile, column
// l%16).  Contractions over a 32-index block use the permuted order
// {4g..4g+3, 16+4g..16+4g+3} for lane group g, which is exactly what two
// stacked accumulator tiles hold, so S, Y and U feed the MFMA B operand from
// registers; the LDS operand planes are stored in that order (pcol), so a
// lane's fragment is one 16-byte read.  Every product uses
// three bf16 MFMAs (hi*hi + hi*lo + lo*hi), i.e. about fp32 accuracy.
// The gated RMSNorm epilogue, checkpoint writes and the final state write are
// fused into the same kernel.

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int CH = 64;       // chunk length
constexpr int RREF = 31;     // reference row of the decay factorisation
// The factorisation through row RREF needs, for every key channel, Gam_RREF
// and Gam_end - Gam_RREF above -FAST_BOUND: every factor then lies in
// [exp(-80), exp(80)], inside the fp32 range.  A chunk uses it when every
// channel's decay over each of its four 16-row blocks stays above
// -FAST_BOUND / 2 (which implies the bound on both halves); other chunks take
// the block-local path (local_planes in prefill_chain).
constexpr float FAST_BOUND = 80.f;
// The block-local path floors each log-decay at -G_FLOOR: exp(-30) = 9.4e-14,
// so what a floored token lets through is below the fp32 resolution of the
// state it multiplies, and the local sums stay finite (a gate of -inf would
// otherwise give -inf - (-inf) in a difference of prefix sums).
constexpr float G_FLOOR = 30.f;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;

struct Frag {
    bf16x8 hi, lo;
};

struct Frag4 {
    bf16x4 hi, lo;
};

__device__ __forceinline__ f32x4 mfma3_16(const Frag4& a, const Frag4& b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, acc, 0, 0, 0);
    return acc;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Split two floats into packed (hi, lo) bf16 pairs with x = hi + lo to about
// 16 significant bits: hi = RNE(x) (one packed conversion for both), lo =
// RNE(x - hi) (x - hi is exact in fp32).
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    const float ha = __uint_as_float(hi << 16), hb = __uint_as_float(hi & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a - ha, b - hb}, bf16x2));
}

union U64 {
    uint2 u;
    bf16x4 v;
};

__device__ __forceinline__ Frag4 split4(const f32x4& x) {
    U64 h, l;
    split2(x[0], x[1], h.u.x, l.u.x);
    split2(x[2], x[3], h.u.y, l.u.y);
    return Frag4{h.v, l.v};
}

// Two 4-element halves stacked into one 8-element operand.
__device__ __forceinline__ Frag cat(const Frag4& a, const Frag4& b) {
    Frag f;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        f.hi[e] = a.hi[e];
        f.hi[e + 4] = b.hi[e];
        f.lo[e] = a.lo[e];
        f.lo[e + 4] = b.lo[e];
    }
    return f;
}

__device__ __forceinline__ f32x4 mfma3(const Frag& a, const Frag& b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    return acc;
}

// Two-term product hi(a) * (hi(b) + lo(b)): b keeps about fp32 accuracy, a is
// rounded once to bf16.  Used where a only feeds the outputs.
__device__ __forceinline__ f32x4 mfma2(const bf16x8& ahi, const Frag& b, f32x4 acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b.hi, acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ Frag split8(const float (&x)[8]) {
    union {
        uint4 u;
        bf16x8 v;
    } h, l;
    split2(x[0], x[1], h.u.x, l.u.x);
    split2(x[2], x[3], h.u.y, l.u.y);
    split2(x[4], x[5], h.u.z, l.u.z);
    split2(x[6], x[7], h.u.w, l.u.w);
    return Frag{h.v, l.v};
}

// A fragment scaled element by element by d and split again into hi/lo.
__device__ __forceinline__ Frag scale_frag(const Frag& f, const float (&d)[8]) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; e++) x[e] = (static_cast<float>(f.hi[e]) + static_cast<float>(f.lo[e])) * d[e];
    return split8(x);
}

__device__ __forceinline__ uint16_t bf16_bits(__bf16 b) { return __builtin_bit_cast(uint16_t, b); }

// Store a at element idx and b at idx + stride of two (hi, lo) planes.
__device__ __forceinline__ void st_split2(uint16_t* hi, uint16_t* lo, int idx, int stride, float a, float b) {
    uint32_t h, l;
    split2(a, b, h, l);
    hi[idx] = static_cast<uint16_t>(h);
    hi[idx + stride] = static_cast<uint16_t>(h >> 16);
    lo[idx] = static_cast<uint16_t>(l);
    lo[idx + stride] = static_cast<uint16_t>(l >> 16);
}

// Rows r and r+1 (values a, b) of one channel into a plane pair whose
// channel c and c+1 (c even) sit side by side, as 32-bit words: the lanes of
// channels c and c+1 (lanes l and l^1) swap half words, the even lane then
// stores row r and the odd lane row r+1 of both channels.  idx is the
// element of (row r, this lane's channel); all lanes of the wave take part.
__device__ __forceinline__ void st_split2_x2(uint16_t* hi, uint16_t* lo, int idx, int stride, float a, float b,
                                            bool odd) {
    uint32_t h, l;
    split2(a, b, h, l);
    const uint32_t ph = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(h), 0xB1, 0xF, 0xF, false));
    const uint32_t pl = static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(l), 0xB1, 0xF, 0xF, false));
    // even: (own row r, partner's row r); odd: (partner's row r+1, own row r+1)
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
    const int at = odd ? idx + stride - 1 : idx;
    *reinterpret_cast<uint32_t*>(hi + at) = __builtin_amdgcn_perm(ph, h, sel);
    *reinterpret_cast<uint32_t*>(lo + at) = __builtin_amdgcn_perm(pl, l, sel);
}

// One element of a plane pair (the lo plane skipped when lo is null).
__device__ __forceinline__ void st_split1(uint16_t* hi, uint16_t* lo, int idx, float a) {
    uint32_t h, l;
    split2(a, 0.f, h, l);
    hi[idx] = static_cast<uint16_t>(h);
    if (lo) lo[idx] = static_cast<uint16_t>(l);
}

// The value hi + lo of one element of a plane pair (exact in fp32).
__device__ __forceinline__ float ld_pair(const uint16_t* hi, const uint16_t* lo, int idx) {
    return __uint_as_float(static_cast<uint32_t>(hi[idx]) << 16) + __uint_as_float(static_cast<uint32_t>(lo[idx]) << 16);
}

union U128 {
    uint4 u;
    bf16x8 v;
};

// 8 consecutive elements [row][k0, k0+8) of a plane pair.
__device__ __forceinline__ Frag ld_nat(const uint16_t* hi, const uint16_t* lo, int off) {
    U128 a, b;
    a.u = *reinterpret_cast<const uint4*>(hi + off);
    b.u = *reinterpret_cast<const uint4*>(lo + off);
    return Frag{a.v, b.v};
}

// The hi plane only of ld_nat.
__device__ __forceinline__ bf16x8 ld_nat_hi(const uint16_t* hi, int off) {
    U128 a;
    a.u = *reinterpret_cast<const uint4*>(hi + off);
    return a.v;
}

// Storage order of the planes that phase B reads as MFMA A operands (K+, Q+
// and K- along dk; P and K-^T along the chunk rows).  Phase B's B operands
// come straight from 16x16 accumulator tiles: lane group g holds rows 4g ..
// 4g+3 of two stacked tiles, that is contraction indices {4g..4g+3,
// 16+4g..16+4g+3} of a group of 32.  Each group of 32 is stored in the order
// that puts those eight side by side -- index 16h + 4g + e at 8g + 4h + e --
// so a lane's A fragment is one 16-byte read.  The intra-chunk products
// contract K+ and Q+ with K- over dk and read both operands in this stored
// order, which pairs the same indices.
__device__ __forceinline__ constexpr int pcol(int j) {
    return (j & ~31) | (((j >> 2) & 3) << 3) | (((j >> 4) & 1) << 2) | (j & 3);
}

// 4 consecutive elements of a plane pair.
__device__ __forceinline__ Frag4 ld4(const uint16_t* hi, const uint16_t* lo, int off) {
    union {
        uint2 u;
        bf16x4 v;
    } a, b;
    a.u = *reinterpret_cast<const uint2*>(hi + off);
    b.u = *reinterpret_cast<const uint2*>(lo + off);
    return Frag4{a.v, b.v};
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Jobs (a, b) = (j >> 2, j & 3) of the intra-chunk block products in the order
// waves take them, one nibble each from the lowest: 0 4 5 8 9 10 12 13 15 14
// 1 2 3 6 7 11 (the six jobs with a < b, which only clear P's upper blocks, last).
constexpr uint64_t kA5Order = 0xB76321EFDCA98540ull;

// A copy of x the optimiser cannot see through.  Lane indices are re-derived
// from such a copy at the start of each phase of the chunk loop, so their
// address arithmetic stays inside the phase instead of being hoisted out of
// the loop and kept live (and spilled) across all of it.
__device__ __forceinline__ int opq(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// An LDS byte offset the optimiser cannot fold into later constants.  LDS
// instructions take a 16-bit immediate offset; with the region bases opaque,
// every access inside a region (all < 64 KiB) uses base register + immediate
// instead of one precomputed address register per access.
__device__ __forceinline__ char* opaque_lds(char* base, uint32_t off) {
    uint32_t v = off;
    asm volatile("" : "+v"(v));
    return base + v;
}

// One activation element through a buffer resource (offsets in bytes).
template <typename ACT>
__device__ __forceinline__ float buf_ld_act(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (sizeof(ACT) == 2) return bf16_to_f32(buf_ld16(r, voff, soff));
    else return buf_ldf(r, voff, soff);
}

template <typename ACT>
__device__ __forceinline__ void buf_st_act(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float x) {
    if constexpr (sizeof(ACT) == 2) buf_st16(r, voff, soff, bf16_bits(static_cast<__bf16>(x)));   // RNE
    else buf_stf(r, voff, soff, x);
}

// One 32-bit word of raw activations starting at channel c (2 bf16 or 1 fp32).
template <typename F>
__device__ __forceinline__ uint32_t pack_word(F&& at, int64_t tok, int c) {
    using T = decltype(at(tok, c));
    if constexpr (sizeof(T) == 2) {
        const T a = at(tok, c), b = at(tok, c + 1);
        return static_cast<uint32_t>(a.bits) | (static_cast<uint32_t>(b.bits) << 16);
    } else {
        return __float_as_uint(at(tok, c));
    }
}

// Store the state tiles of one 16-column strip (accumulator layout) into a
// dk x dv fp32 state at dst.
template <int IB, int DV>
__device__ __forceinline__ void store_state_strip(float* dst, const f32x4 (&S)[IB], int g4, int jcol, int dk) {
    const auto rs = make_rsrc(dst, static_cast<uint32_t>(dk * DV * 4));
    const uint32_t sv = static_cast<uint32_t>((4 * g4 * DV + jcol) * 4);
#pragma unroll
    for (int ib = 0; ib < IB; ib++)
#pragma unroll
        for (int e = 0; e < 4; e++) buf_stf(rs, sv, (16 * ib + e) * DV * 4, S[ib][e]);
}

// The strip stored in the state dtype of a pool (fp32, or bf16 rounded to
// nearest even).  With a bf16 pool the chain continues from the stored
// value: S is rounded in place.
template <int IB, int DV>
__device__ __forceinline__ void store_pool_strip(void* pool, int64_t slot_head, f32x4 (&S)[IB], int g4, int jcol,
                                                 int dk, bool bf16) {
    if (!bf16) {
        store_state_strip<IB, DV>(static_cast<float*>(pool) + slot_head * dk * DV, S, g4, jcol, dk);
        return;
    }
    const auto rs = make_rsrc(static_cast<uint16_t*>(pool) + slot_head * dk * DV, static_cast<uint32_t>(dk * DV * 2));
    const uint32_t sv = static_cast<uint32_t>((4 * g4 * DV + jcol) * 2);
#pragma unroll
    for (int ib = 0; ib < IB; ib++)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{S[ib][e], S[ib][e + 1]}, bf16x2));
            buf_st16(rs, sv, (16 * ib + e) * DV * 2, static_cast<uint16_t>(w));
            buf_st16(rs, sv, (16 * ib + e + 1) * DV * 2, static_cast<uint16_t>(w >> 16));
            S[ib][e] = __uint_as_float(w << 16);
            S[ib][e + 1] = __uint_as_float(w & 0xffff0000u);
        }
}

// Registers holding one chunk's staged inputs between the loads and the LDS
// stores: raw q|k|v rows (with 3 rows of left context) as 16-byte words, this
// thread's 16 log-decay values, and (threads 0..63) one beta.
template <int NU>
struct Staged {
    uint4 val[NU];
    float gq[16];
    float beta;
};

// Which 16-byte unit of the raw rows a staging slot covers.  Slots are
// grouped per wave so that one wave's slot j always reads one tensor (q, k or
// v): its loads then take a single buffer resource.  A tensor's units are the
// (CH+3) x (D/VEC) 16-byte pieces of its rows (3 rows of left context first).
template <typename ACT, int D, int NT, int NTEN = 3>
struct StageMap {
    static constexpr int VEC = 16 / static_cast<int>(sizeof(ACT));
    static constexpr int UPT = D / VEC;                    // units per tensor row
    static constexpr int UT = (CH + 3) * UPT;              // units per tensor
    static constexpr int WS = (UT + 63) / 64;              // wave slots per tensor
    static constexpr int NWV = NT / 64;
    static constexpr int NU = (NTEN * WS + NWV - 1) / NWV; // slots per thread (NTEN tensors: q, k[, v])
    struct Unit {
        int tensor;   // 0 q, 1 k, 2 v; 3 = unused slot
        int r, col;   // row (0 = three tokens before the chunk), first channel
        bool valid;
    };
    __device__ static Unit unit(int j, int wv, int lane) {
        const int w = j * NWV + wv;
        const int local = (w % WS) * 64 + lane;
        Unit u;
        u.tensor = w / WS;
        u.r = local / UPT;
        u.col = (local % UPT) * VEC;
        u.valid = u.tensor < NTEN && local < UT;
        return u;
    }
};

// Issue the global loads of the chunk [tc0, tc0+n) of head h (no waits): the
// raw q, k (and v) rows (ROWS) and the log-decays and beta (GATES), which a
// caller may request at different points.  Left-context rows before the
// sequence start (first packed token ctx0) come from the initial conv state
// x0 (index 2 = the token just before the start).
template <typename ACT, int DK, int DV, int NT, int NTEN, bool ROWS = true, bool GATES = true, int NU>
__device__ __forceinline__ void stage_issue(Staged<NU>& st, const PrefillParams& p, const ACT* x0,
                                            int64_t ctx0, int64_t tc0, int n, int H, int h, int tp) {
    static_assert(DK == DV, "one row layout for q, k and v");
    using M = StageMap<ACT, DK, NT, NTEN>;
    static_assert(M::NU == NU, "staging slots");
    if constexpr (ROWS) {
        constexpr int D = DK;
        const int wv = __builtin_amdgcn_readfirstlane(tp >> 6), lane = tp & 63;
        // resources start at the first row inside the sequence; rows before it
        // (and rows past the chunk) fall outside and read as zero
        const int64_t first = max(tc0 - 3, ctx0);
        const int d0 = static_cast<int>(first - (tc0 - 3));                // 0..3 rows of context from x0
        const int64_t hoff = (first * H + h) * D;
        const uint32_t nbytes = static_cast<uint32_t>(((tc0 + n - 1 - first) * H + 1) * D * sizeof(ACT));
        const uint32_t rowb = static_cast<uint32_t>(H * D * sizeof(ACT));
        const ACT* tens[3] = {static_cast<const ACT*>(p.q), static_cast<const ACT*>(p.k), static_cast<const ACT*>(p.v)};
#pragma unroll
        for (int j = 0; j < NU; j++) {
            const typename M::Unit u = M::unit(j, wv, lane);
            st.val[j] = make_uint4(0, 0, 0, 0);
            const int tsel = __builtin_amdgcn_readfirstlane(u.tensor);
            if (tsel < NTEN) {
                const auto rs = make_rsrc(tens[tsel] + hoff, nbytes);
                const int rel = u.r - d0;
                const uint32_t vo = (u.valid && rel >= 0) ? static_cast<uint32_t>(rel) * rowb + u.col * sizeof(ACT)
                                                          : 0x80000000u;
                const float4 x = buf_ld4(rs, vo, 0);
                st.val[j] = make_uint4(__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z),
                                       __float_as_uint(x.w));
            }
        }
        if (d0 > 0) {
            // context rows before the sequence start: raw values from x0
#pragma unroll
            for (int j = 0; j < NU; j++) {
                const typename M::Unit u = M::unit(j, wv, lane);
                if (u.valid && u.r < d0) {
                    const int m = 3 - d0 + u.r;                 // x0 index of this token
                    const int c0 = u.tensor * D + u.col;
                    uint32_t wd[4];
#pragma unroll
                    for (int q4 = 0; q4 < 4; q4++) {
                        const int c = c0 + q4 * (M::VEC / 4);
                        if constexpr (sizeof(ACT) == 2) {
                            wd[q4] = static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(x0)[c * 3 + m]) |
                                     (static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(x0)[(c + 1) * 3 + m]) << 16);
                        } else {
                            wd[q4] = __float_as_uint(reinterpret_cast<const float*>(x0)[c * 3 + m]);
                        }
                    }
                    st.val[j] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
                }
            }
        }
    }
    if constexpr (GATES) {
        // row t of this head at byte offset t * row_bytes; the resources end after
        // row n-1 and the whole offset is in the range-checked per-lane offset, so
        // rows past the chunk read as zero
        const int cgp = tp % DK, qqp = tp / DK;
        const auto rg = make_rsrc(p.g + (tc0 * H + h) * DK, static_cast<uint32_t>(((n - 1) * H + 1) * DK * 4));
        const uint32_t gv = static_cast<uint32_t>((16 * qqp * H * DK + cgp) * 4);
#pragma unroll
        for (int r = 0; r < 16; r++) st.gq[r] = buf_ldf(rg, gv + static_cast<uint32_t>(r * H * DK * 4), 0);
        st.beta = 0.f;
        if (tp < CH) {
            const auto rb = make_rsrc(p.beta + tc0 * H + h, static_cast<uint32_t>(((n - 1) * H + 1) * 4));
            st.beta = buf_ldf(rb, static_cast<uint32_t>(tp * H * 4), 0);
        }
    }
}

// Define every staged register without loading (after the last chunk), so
// that no value of the previous chunk stays live across the loop.
template <int NU>
__device__ __forceinline__ void stage_clear(Staged<NU>& st) {
#pragma unroll
    for (int j = 0; j < NU; j++) st.val[j] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; r++) st.gq[r] = 0.f;
    st.beta = 0.f;
}

// Store the staged raw rows and beta into LDS (rows of CR elements: q, k, v).
template <typename ACT, int DK, int DV, int NT, int NTEN, int NU>
__device__ __forceinline__ void stage_commit(const Staged<NU>& st, ACT* raw, float* beta_s, int tp) {
    using M = StageMap<ACT, DK, NT, NTEN>;
    constexpr int C = 2 * DK + DV;
    constexpr int CR = C + M::VEC;              // padded row stride (spreads the v reads of the conv over banks)
    const int wv = __builtin_amdgcn_readfirstlane(tp >> 6), lane = tp & 63;
#pragma unroll
    for (int j = 0; j < NU; j++) {
        const typename M::Unit u = M::unit(j, wv, lane);
        if (u.valid) *reinterpret_cast<uint4*>(raw + u.r * CR + u.tensor * DK + u.col) = st.val[j];
    }
    if (tp < CH) beta_s[tp] = st.beta;
}

template <int D, typename ACT>
struct PrefillShape {
    static constexpr int DK = D, DV = D;
    static constexpr int NW = DV / 16;          // waves = 16-column strips of S
    static constexpr int NT = 64 * NW;
    static constexpr int C = 2 * DK + DV;       // conv channels
    static constexpr int KS = DK / 32;          // 32-channel contraction steps
    static constexpr int IB = DK / 16;          // 16-row tiles of S
    static constexpr int PS = DK + 8;           // padded row stride of [64][dk] planes
    static constexpr int QS = CH + 8;           // padded row stride of [*][64] planes
    static constexpr int VEC = 16 / static_cast<int>(sizeof(ACT));   // elements per 16-byte load
    static constexpr int CR = C + VEC;          // padded row stride of the raw rows
    static constexpr int FP = DK + 4;           // padded row stride of the fp32 q/k planes
    // LDS regions (bytes)
    static constexpr int R0 = cmax(CH * FP * 4, 2 * CH * PS * 2);                // a_k (fp32) / K+ planes
    static constexpr int R1 = R0;                                                 // a_q (fp32) / Q+ planes
    static constexpr int R2 = cmax(2 * CH * PS * 2, 2 * DK * QS * 2);           // K- planes / K-^T planes
    static constexpr int R4 = 2 * CH * QS * 2;                                   // L planes, T_aa on the diagonal
    static constexpr int R5 = 2 * CH * QS * 2;                                   // P planes
    static constexpr int RAW = (CH + 3) * CR * static_cast<int>(sizeof(ACT));   // raw rows (aliases R2..R5)
    static constexpr int O0 = 0, O1 = R0, O2 = 2 * R0, O4 = O2 + R2, O5 = O4 + R4;
    static constexpr int BYTES = O5 + R5;
    static_assert(RAW <= R2 + R4 + R5, "raw staging must fit in the aliased regions");
    static_assert(NT / (2 * DK) == 2 && NT / DK == 4, "thread mappings assume nt = 4 * dk");
};

// Shared memory of one chain's workgroup.  sv holds what phase A hands to
// phase B besides the planes: beta, exp(Gam_r), exp(Gam_end) and
// exp(Gam_end - Gam_r) per key channel.
template <int D, typename ACT>
struct PrefillLds {
    using Sh = PrefillShape<D, ACT>;
    __attribute__((aligned(16))) char lds[Sh::BYTES];
    __attribute__((aligned(16))) float sv[CH + 3 * D];
    float rq[CH], rk[CH];
    float gtot[4][D];
    float part[Sh::NW][CH];
    float rinv[CH];
    float ld[4][16][16];       // diagonal blocks of L (fp32)
    ACT x0[Sh::C * 3];
    ACT vwin[sizeof(ACT) == 2 ? 1 : (CH + 3) * D];   // consumer's raw v rows (fp32 activations)
    int flag;
    int local;                 // the chunk takes the block-local decay path
    int early;                 // consumer: this chunk's slot was requested during the previous epilogue
};

// A thread's 16 consecutive entries of K-^T row c (chunk rows 16 qq ..
// 16 qq + 15) into the hi/lo planes, in pcol order: four 8-byte stores per
// plane, at 8g + 4 (qq & 1) of the row's group of 32 for rows 4g .. 4g + 3.
template <int QS>
__device__ __forceinline__ void st_kt(uint16_t* kt_h, uint16_t* kt_l, int c, int qq, const float (&km)[16]) {
    uint32_t wh[8], wl[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) split2(km[r], km[r + 1], wh[r / 2], wl[r / 2]);
    const int o = c * QS + pcol(16 * qq);
#pragma unroll
    for (int g = 0; g < 4; g++) {
        *reinterpret_cast<uint2*>(kt_h + o + 8 * g) = make_uint2(wh[2 * g], wh[2 * g + 1]);
        *reinterpret_cast<uint2*>(kt_l + o + 8 * g) = make_uint2(wl[2 * g], wl[2 * g + 1]);
    }
}

// Roles of a chain's workgroup.  FUSED runs both phases of every chunk.  In a
// pair, a PRODUCER runs phase A of every chunk of its chain (without v's
// conv) and hands the chunk's planes and sv to its CONSUMER through a ring of
// RING slots in the workspace; the consumer convolves v, runs phase B, the
// epilogue, checkpoints and the final state.  The arithmetic is the fused
// code itself, so a paired chain gives the fused run's bits.
constexpr int FUSED = 0, PRODUCER = 1, CONSUMER = 2;
constexpr int RING = 3;

// Bytes of one ring slot: the LDS planes, then sv.
template <int D, typename ACT>
constexpr int64_t pair_slot_bytes() {
    using Sh = PrefillShape<D, ACT>;
    return (static_cast<int64_t>(Sh::BYTES) + (CH + 3 * D) * 4 + 255) / 256 * 256;
}

// Ring words are stored and loaded with the device-coherent cache policy
// (SC1, the policy of device-scope atomics on gfx950): a store is visible to
// such loads from every XCD once it has completed, so no L2 write-back or
// invalidate (a device-scope fence) is needed.  A producer makes every
// thread wait for its stores to complete, meets at a barrier, and only then
// moves the chunk counter; a consumer loads only after it has seen the counter.
constexpr int RING_POL = 16;   // SC1 bit of the buffer cache-policy operand
constexpr int VMCNT0 = 0x0F70;  // s_waitcnt operand: vector memory count 0, the other counters untouched

__device__ __forceinline__ uint4 ring_ld(__amdgpu_buffer_rsrc_t r, uint32_t word) {
    const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(word * 16), 0, RING_POL);
    return make_uint4(static_cast<uint32_t>(v.x), static_cast<uint32_t>(v.y), static_cast<uint32_t>(v.z),
                      static_cast<uint32_t>(v.w));
}
__device__ __forceinline__ void ring_st(__amdgpu_buffer_rsrc_t r, uint32_t word, uint4 x) {
    i32x4 v;
    v.x = static_cast<int>(x.x);
    v.y = static_cast<int>(x.y);
    v.z = static_cast<int>(x.z);
    v.w = static_cast<int>(x.w);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(word * 16), 0, RING_POL);
}

// Store NW 16-byte words of LDS into a ring slot (from word w0 on), word e
// by thread e % NT, NB LDS reads at a time ahead of their stores.
template <int NW, int NT, int NB>
__device__ __forceinline__ void ring_put(__amdgpu_buffer_rsrc_t r, uint32_t w0, const uint4* lds_words, int tp) {
    constexpr int FULL = NW / NT, REM = NW % NT;
#pragma unroll
    for (int b = 0; b < FULL; b += NB) {
        uint4 w[NB];
#pragma unroll
        for (int i = 0; i < NB; i++)
            if (b + i < FULL) w[i] = lds_words[(b + i) * NT + tp];
#pragma unroll
        for (int i = 0; i < NB; i++)
            if (b + i < FULL) ring_st(r, w0 + (b + i) * NT + tp, w[i]);
    }
    if (REM > 0 && tp < REM) ring_st(r, w0 + FULL * NT + tp, lds_words[FULL * NT + tp]);
}

// Load two word ranges of a ring slot, [0, NA) and [B0, B0 + NB), into the
// same words of LDS: every load is issued before the first LDS store, so the
// whole copy costs one memory round trip.
template <int NA, int B0, int NB, int NT>
__device__ __forceinline__ void ring_get2(__amdgpu_buffer_rsrc_t r, uint4* lds_words, int tp) {
    constexpr int FA = NA / NT, RA = NA % NT, FB = NB / NT, RB = NB % NT;
    uint4 wa[FA + 1], wb[FB + 1];
#pragma unroll
    for (int i = 0; i < FA; i++) wa[i] = ring_ld(r, i * NT + tp);
    if (RA > 0 && tp < RA) wa[FA] = ring_ld(r, FA * NT + tp);
#pragma unroll
    for (int i = 0; i < FB; i++) wb[i] = ring_ld(r, B0 + i * NT + tp);
    if (RB > 0 && tp < RB) wb[FB] = ring_ld(r, B0 + FB * NT + tp);
#pragma unroll
    for (int i = 0; i < FA; i++) lds_words[i * NT + tp] = wa[i];
    if (RA > 0 && tp < RA) lds_words[FA * NT + tp] = wa[FA];
#pragma unroll
    for (int i = 0; i < FB; i++) lds_words[B0 + i * NT + tp] = wb[i];
    if (RB > 0 && tp < RB) lds_words[B0 + FB * NT + tp] = wb[FB];
}

// One 16-byte word per lane from a buffer straight into LDS with the ring's
// device-coherent policy (buffer load with the LDS bit: lane l writes LDS
// bytes [lds + 16 l, lds + 16 l + 16), so a wave instruction fills 64
// consecutive words; no register holds the data).  The copy is asynchronous:
// the wave waits for its vector memory count to drain, and the workgroup
// meets at a barrier, before anyone reads the words.  Written as inline
// assembly so that the compiler, which cannot tell which LDS bytes such a
// copy writes, does not make unrelated LDS reads wait for it.
__device__ __forceinline__ void ring_word_to_lds(i32x4 rsrc, uint32_t lds, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen sc1 lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
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

__device__ __forceinline__ uint32_t lds_addr(void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(p)));
}

// One 16-byte word of an input tensor per lane into LDS (M0 = the wave's
// 1 KiB destination, lane l at + 16 l), no registers; an offset outside the
// resource reads as zero.
__device__ __forceinline__ void input_word_to_lds(i32x4 rsrc, uint32_t lds, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// A consumer's raw v rows of the chunk [tc0, tc0 + n): CH + 3 rows of DV
// values in vwin (row 0 is three tokens before the chunk), copied straight
// from global memory into LDS, 16-byte word u by lane u % 64 of wave
// (u / 64) % NWV.  Rows before the sequence start (packed index ctx0) and
// rows past the chunk read as zero; the former are filled from the initial
// conv state by vwin_fix once the copy has landed, the latter only feed
// masked rows.  Complete after the issuing wave's vmcnt(0) and a barrier.
template <typename ACT, int DV, int NWV>
__device__ __forceinline__ void vwin_copy(const PrefillParams& p, ACT* vwin, int64_t ctx0, int64_t tc0, int n,
                                          int H, int h, int wave, int lane) {
    constexpr int VEC = 16 / static_cast<int>(sizeof(ACT));
    constexpr int UPR = DV / VEC;                      // words per row
    constexpr int UNITS = (CH + 3) * UPR;
    const int64_t first = max(tc0 - 3, ctx0);
    const int d0 = static_cast<int>(first - (tc0 - 3));
    i32x4 r = raw_rsrc(static_cast<const ACT*>(p.v) + (first * H + h) * DV,
                       static_cast<uint32_t>(((tc0 + n - 1 - first) * H + 1) * DV * sizeof(ACT)));
#pragma unroll
    for (int i = 0; i < 4; i++) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
    const uint32_t lv = __builtin_amdgcn_readfirstlane(lds_addr(vwin));
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t rowb = static_cast<uint32_t>(H * DV * sizeof(ACT));
#pragma unroll 1
    for (int b = wv; b < (UNITS + 63) / 64; b += NWV) {
        const int u = 64 * b + lane, row = u / UPR, col = (u % UPR) * VEC;
        const uint32_t vo = row >= d0 ? static_cast<uint32_t>(row - d0) * rowb + col * sizeof(ACT) : 0x80000000u;
        if (u < UNITS) input_word_to_lds(r, lv + 1024 * b, vo);
    }
}

// Rows of vwin before the sequence start, from the initial conv state x0
// (after the copy has landed: its zeros would overwrite them).
template <typename ACT, int DK, int DV, int NT>
__device__ __forceinline__ void vwin_fix(ACT* vwin, const ACT* x0, int64_t ctx0, int64_t tc0, int tp) {
    const int d0 = static_cast<int>(max(tc0 - 3, ctx0) - (tc0 - 3));
    for (int e = tp; e < d0 * DV; e += NT) {
        const int r = e / DV, c = e % DV;
        vwin[r * DV + c] = x0[(2 * DK + c) * 3 + 3 - d0 + r];
    }
}

// The words ring_get2 loads ([0, NA) and [B0, B0 + NB)) and the NS sv words
// from word S0 on, copied into LDS as ring_word_to_lds does: each wave takes
// every NWV-th block of 64 words; lanes outside the ranges write nothing.
// The resource, the LDS bases and the wave index are made wave-uniform
// (scalar registers), as the copy's scalar operands must be.
template <int NA, int B0, int NB, int NS, int S0, int NWV>
__device__ __forceinline__ void ring_get2_async(const void* slot, uint32_t slot_bytes, void* planes, void* sv,
                                                int wave, int lane) {
    i32x4 r = raw_rsrc(slot, slot_bytes);
#pragma unroll
    for (int i = 0; i < 4; i++) r[i] = __builtin_amdgcn_readfirstlane(r[i]);
    const uint32_t lp = __builtin_amdgcn_readfirstlane(lds_addr(planes));
    const uint32_t ls = __builtin_amdgcn_readfirstlane(lds_addr(sv));
    const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll 1
    for (int b = wv; b < (NA + 63) / 64; b += NWV) {
        const int w = 64 * b + lane;
        if (w < NA) ring_word_to_lds(r, lp + 1024 * b, 16 * w);
    }
#pragma unroll 1
    for (int b = B0 / 64 + wv; b < (B0 + NB + 63) / 64; b += NWV) {
        const int w = 64 * b + lane;
        if (w >= B0 && w < B0 + NB) ring_word_to_lds(r, lp + 1024 * b, 16 * w);
    }
#pragma unroll 1
    for (int b = wv; b < (NS + 63) / 64; b += NWV) {
        const int w = 64 * b + lane;
        if (w < NS) ring_word_to_lds(r, ls + 1024 * b, 16 * (S0 + w));
    }
}

// A ring counter read ahead of need (one lane): the read takes a memory round
// trip, so it is issued well before the value is needed.
__device__ __forceinline__ int ring_peek(const int32_t* ctr) {
    return __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until a ring counter reaches want (one lane), given a value read
// earlier: only when that value falls short is the counter polled, at most
// `limit` times (each poll sleeps 128 cycles).  A wait that runs out means
// the partner is gone; it is counted in the call's status word.
__device__ __forceinline__ bool ring_wait(const int32_t* ctr, int want, int seen, int limit, int32_t* status) {
    if (seen >= want) return true;
    for (int it = 0; it < limit; it++) {
        if (ring_peek(ctr) >= want) return true;
        __builtin_amdgcn_s_sleep(2);
    }
    __hip_atomic_fetch_add(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
}

// One (sequence, head) chain, or one segment of it, in the given role.
// OUT: outputs, checkpoints and final states of whole sequences or segments.
// !OUT (segment transitions, FUSED only): the segment's end state from a
// zero state (G) and its transition matrix (F: the state propagated from the
// identity with v = 0), side by side, sharing each chunk's state-independent
// part.
// CD (conv done): q, k and v each hold two tensors back to back, the
// activations after the causal conv and SiLU (what phase A would compute
// from the raw inputs, rounded to bf16) and the raw inputs; phase A then
// takes the activations as they are, and the conv states written at
// checkpoints and at the end still come from the raw inputs.
template <int D, typename ACT, bool OUT, int ROLE, bool CD = false>
__device__ __forceinline__ void prefill_chain(const PrefillParams& p, PrefillLds<D, ACT>& sm, int item, const int h) {
    static_assert(ROLE == FUSED || OUT, "paired roles produce outputs");
    using Sh = PrefillShape<D, ACT>;
    constexpr int DK = Sh::DK, DV = Sh::DV, NW = Sh::NW, NT = Sh::NT, C = Sh::C;
    constexpr int KS = Sh::KS, IB = Sh::IB, PS = Sh::PS, QS = Sh::QS, VEC = Sh::VEC;
    constexpr int CR = Sh::CR, FP = Sh::FP;
    using A = Act<ACT>;
    // With bf16 outputs the output-only products (Q_g S, P U) take the LDS
    // operand in one bf16 term; fp32 outputs keep three terms everywhere.
    constexpr bool kOutHi = sizeof(ACT) == 2;

    char* const lds = sm.lds;
    float* const beta_s = sm.sv;
    float* const eGr_s = sm.sv + CH;
    float* const eGC_s = sm.sv + CH + DK;
    float* const eGCr_s = sm.sv + CH + 2 * DK;
    float (&rq_s)[CH] = sm.rq;
    float (&rk_s)[CH] = sm.rk;
    float (&gtot_s)[4][DK] = sm.gtot;
    float (&part_s)[NW][CH] = sm.part;
    float (&rinv_s)[CH] = sm.rinv;
    float (&ld_s)[4][16][16] = sm.ld;
    ACT (&x0_s)[C * 3] = sm.x0;

    char* reg0 = opaque_lds(lds, Sh::O0);
    char* reg1 = opaque_lds(lds, Sh::O1);
    char* reg2 = opaque_lds(lds, Sh::O2);
    char* reg4 = opaque_lds(lds, Sh::O4);
    char* reg5 = opaque_lds(lds, Sh::O5);
    float* ak_f = reinterpret_cast<float*>(reg0);                // [CH][FP] fp32
    float* aq_f = reinterpret_cast<float*>(reg1);
    // transition pass (no outputs, so no q): SiLU(conv(v)) of each thread,
    // [16][NT] fp32, from phase A to phase B where the Q+ planes would be
    float* vst = reinterpret_cast<float*>(reg1);
    static_assert(16 * NT * 4 <= Sh::R1, "the v values fit in the Q+ region");
    uint16_t* kp_h = reinterpret_cast<uint16_t*>(reg0);          // K+ planes [CH][PS]
    uint16_t* kp_l = kp_h + CH * PS;
    uint16_t* qp_h = reinterpret_cast<uint16_t*>(reg1);          // Q+ planes
    uint16_t* qp_l = qp_h + CH * PS;
    uint16_t* km_h = reinterpret_cast<uint16_t*>(reg2);          // K- planes [CH][PS]
    uint16_t* km_l = km_h + CH * PS;
    uint16_t* kt_h = reinterpret_cast<uint16_t*>(reg2);          // K-^T planes [DK][QS]
    uint16_t* kt_l = kt_h + DK * QS;
    uint16_t* lp_h = reinterpret_cast<uint16_t*>(reg4);          // L planes [CH][QS], T_aa on the diagonal
    uint16_t* lp_l = lp_h + CH * QS;
    uint16_t* pp_h = reinterpret_cast<uint16_t*>(reg5);          // P planes [CH][QS]
    uint16_t* pp_l = pp_h + CH * QS;
    ACT* raw = reinterpret_cast<ACT*>(reg2);                     // [CH+3][CR]
    // consumer: raw v rows [CH+3][DV]; with bf16 outputs phase B never reads
    // the Q+ lo plane, whose region holds them
    ACT* vwin = kOutHi ? reinterpret_cast<ACT*>(qp_l) : sm.vwin;
    static_assert(!kOutHi || (CH + 3) * DV * static_cast<int>(sizeof(ACT)) <= Sh::R1 - CH * PS * 2,
                  "the v rows fit in the Q+ lo plane");
    // 16-byte words of a ring slot: the planes phase B reads, K+ and Q+ (words
    // [0, NPA)), K-^T, L and P (words [PB0, PB0 + NPB)) -- with bf16 outputs
    // phase B reads only the hi planes of Q+ and P -- then sv (NSV words
    // from NPW on)
    constexpr int NPW = Sh::BYTES / 16;
    constexpr int NPA = (Sh::O1 + (kOutHi ? CH * PS * 2 : Sh::R1)) / 16;
    constexpr int PB0 = Sh::O2 / 16;
    constexpr int NPB = (Sh::O5 + (kOutHi ? CH * QS * 2 : Sh::R5)) / 16 - PB0;
    static_assert(Sh::BYTES % 16 == 0 && Sh::O1 % 16 == 0 && Sh::O2 % 16 == 0 && Sh::O5 % 16 == 0 &&
                  (CH * PS * 2) % 16 == 0 && (CH * QS * 2) % 16 == 0, "16-byte plane words");
    constexpr int NSV = (CH + 3 * DK) / 4;
    static_assert(NSV <= NT, "one sv word per thread");

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, l16 = lane & 15;
    const int H = p.H;
    const SeqWork wk = p.work[item];
    if (wk.len < 0) return;                    // malformed sequence bounds or unused item: nothing is touched
    if constexpr (!OUT) {
        if (wk.last) return;                   // the last segment of a sequence needs no transition
    }
    const int seq = wk.seq;
    const int64_t tok0 = wk.tok0;
    const int64_t ctx0 = wk.ctx0;
    const int L = wk.len;
    const int64_t start = wk.start;
    const int init = p.init_slot ? p.init_slot[seq] : -1;
    const int fin = (p.final_slot && wk.last) ? p.final_slot[seq] : -1;   // only the last item writes it
    const int jcol = 16 * wave + l16;          // this lane's state / output column
    // Segments of a split sequence take their initial state and conv state from
    // the workspace, filled before this launch: a final slot that is also the
    // initial slot is then only written after every read of it.
    const bool seg_in = OUT && p.split && !(wk.part == 0 && wk.last);

    // invalid initial slot or position: NaN outputs, no state written
    if (init < -1 || init >= p.num_slots || start < 0) {
        if constexpr (OUT && ROLE != PRODUCER) {
            for (int64_t e = tid; e < static_cast<int64_t>(L) * DV; e += NT) {
                const int64_t t = tok0 + e / DV;
                A::st(static_cast<ACT*>(p.out) + (t * H + h) * DV + e % DV, nan_f32());
            }
        }
        return;
    }

    // ---- chain prologue: initial state (accumulator layout), conv state, weights
    f32x4 S[IB];
    f32x4 SF[OUT ? 1 : IB];    // F's strip (transition pass only)
    {
        const uint32_t sv = static_cast<uint32_t>((4 * g4 * DV + jcol) * 4);
        const float* s0 = nullptr;          // fp32 source
        const uint16_t* s0h = nullptr;      // bf16 source
        if constexpr (OUT) {
            const int64_t ih = (static_cast<int64_t>(init) * H + h) * DK * DV;
            if (seg_in) s0 = p.seg_S + (static_cast<int64_t>(item) * H + h) * DK * DV;
            else if (init >= 0 && p.state_bf16) s0h = static_cast<const uint16_t*>(p.state) + ih;
            else if (init >= 0) s0 = static_cast<const float*>(p.state) + ih;
        }
        if (s0) {
            const auto rs = make_rsrc(s0, DK * DV * 4);
#pragma unroll
            for (int ib = 0; ib < IB; ib++)
#pragma unroll
                for (int e = 0; e < 4; e++) S[ib][e] = buf_ldf(rs, sv, (16 * ib + e) * DV * 4);
        } else if (s0h) {
            const auto rs = make_rsrc(s0h, DK * DV * 2);
#pragma unroll
            for (int ib = 0; ib < IB; ib++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    S[ib][e] = __uint_as_float(static_cast<uint32_t>(buf_ld16(rs, sv / 2, (16 * ib + e) * DV * 2)) << 16);
        } else {
#pragma unroll
            for (int ib = 0; ib < IB; ib++)
#pragma unroll
                for (int e = 0; e < 4; e++) S[ib][e] = 0.f;
        }
        if constexpr (!OUT) {
#pragma unroll
            for (int ib = 0; ib < IB; ib++)
#pragma unroll
                for (int e = 0; e < 4; e++) SF[ib][e] = 16 * ib + 4 * g4 + e == jcol ? 1.f : 0.f;
        }
        const int64_t hx = (static_cast<int64_t>(seq) * H + h) * C * 3;
        const ACT* x0 = seg_in ? static_cast<const ACT*>(p.seq_x0) + hx
                               : (init >= 0 ? static_cast<const ACT*>(p.conv) + (static_cast<int64_t>(init) * H + h) * C * 3
                                            : nullptr);
        // the zero-start pass of a sequence's first segment keeps its initial
        // conv state for the segments' output pass
        ACT* keep = (!OUT && wk.part == 0) ? static_cast<ACT*>(p.seq_x0) + hx : nullptr;
        for (int e = tid; e < C * 3; e += NT) {
            if (x0) x0_s[e] = x0[e];
            else A::st(&x0_s[e], 0.f);
            if (keep) keep[e] = x0_s[e];
        }
    }
    const int cqk = tid % (2 * DK);                              // q/k conv channel of this thread
    const float4 wqk = *reinterpret_cast<const float4*>(p.conv_w + (static_cast<int64_t>(h) * C + cqk) * 4);
    const float4 wv = *reinterpret_cast<const float4*>(p.conv_w + (static_cast<int64_t>(h) * C + 2 * DK + jcol) * 4);
    const float nwj = p.norm_w[jcol];
    // raw inputs (the conv state's contents): with CD, the second tensor of each pair
    const ACT* qin = static_cast<const ACT*>(p.q) + (CD ? p.T * H * DK : 0);
    const ACT* kin = static_cast<const ACT*>(p.k) + (CD ? p.T * H * DK : 0);
    const ACT* vin = static_cast<const ACT*>(p.v) + (CD ? p.T * H * DV : 0);
    const ACT* zin = static_cast<const ACT*>(p.z);
    ACT* out = static_cast<ACT*>(p.out);
    __syncthreads();

    // raw input value of channel c at packed token tok (conv left context)
    auto raw_at = [&](int64_t tok, int c) -> ACT {
        if (tok >= ctx0) {
            const ACT* src = c < DK ? qin + (tok * H + h) * DK + c
                                    : (c < 2 * DK ? kin + (tok * H + h) * DK + (c - DK)
                                                  : vin + (tok * H + h) * DV + (c - 2 * DK));
            return *src;
        }
        return x0_s[c * 3 + 3 - static_cast<int>(ctx0 - tok)];
    };
    // conv state after the tokens before packed index tend: the last 3 raw inputs
    auto write_conv_state = [&](ACT* dst, int64_t tend) {
        for (int e = tid; e < C * 3; e += NT) {
            const int c = e / 3, m = e % 3;
            dst[e] = raw_at(tend - 3 + m, c);
        }
    };
    int64_t pos = start;
    // paired roles: this chain's ring slots and its two counters (chunks
    // handed over, chunks taken)
    const int64_t chain = static_cast<int64_t>(item) * H + h;
    char* const ring = ROLE == FUSED ? nullptr : p.ring + chain * RING * pair_slot_bytes<D, ACT>();
    int32_t* const ready_ctr = ROLE == FUSED ? nullptr : p.ring_ctr + chain * 32;
    int32_t* const taken_ctr = ROLE == FUSED ? nullptr : p.ring_ctr + chain * 32 + 16;
    int chunk = 0;
    int seen = 0;       // thread 0 of a paired role: the partner's counter as last read
    // checkpoint counter: a segment that ends at a checkpoint position leaves
    // that checkpoint to the next segment (which starts from the scanned
    // state), so a segment that is not the last of its sequence writes none
    int done = 0, ck = wk.last ? wk.part : -(1 << 30);
    // (clamped so that adding a checkpoint index cannot overflow; no slot lies
    // outside the clamp range)
    const int ck_base = (OUT && p.ckpt_interval > 0) ? min(max(p.ckpt_base[seq], -(1 << 30)), 1 << 30) : 0;
    if constexpr (OUT && ROLE != PRODUCER) {
        // a segment after the first starts at a checkpoint position: its
        // initial state (from the scan of the segment transitions) is that
        // checkpoint
        if (p.ckpt_interval > 0 && wk.part > 0) {
            const int slot = ck_base + wk.part - 1;
            if (slot >= 0 && slot < p.num_ckpt_slots) {
                const int64_t sh = static_cast<int64_t>(slot) * H + h;
                store_pool_strip<IB, DV>(p.ckpt_state, sh, S, g4, jcol, DK, p.state_bf16);
                write_conv_state(static_cast<ACT*>(p.ckpt_conv) + sh * C * 3, tok0);
            }
        }
    }

    // ---------------- A1 of the first chunk (later chunks are staged while the
    // previous chunk finishes: their loads are issued after its state phase)
    // the producer stages q and k only: v rows are read by the consumer
    constexpr int NTEN = ROLE == PRODUCER ? 2 : 3;
    Staged<StageMap<ACT, D, NT, NTEN>::NU> stg;
    int n = L > 0 ? min(L, CH - static_cast<int>(pos % CH)) : 0;
    int64_t tc0 = tok0;
    if (ROLE != CONSUMER && L > 0) {
        const int tp = opq(tid);
        stage_issue<ACT, DK, DV, NT, NTEN>(stg, p, x0_s, ctx0, tc0, n, H, h, tp);
        stage_commit<ACT, DK, DV, NT, NTEN>(stg, raw, beta_s, tp);
    }
    if (tid == 0) {
        sm.local = 0;
        sm.early = 0;
    }
    __syncthreads();

    // ---- block-local decay path, for chunks whose decay leaves the range of
    // the factorisation through row RREF.  Every pairwise factor
    // exp(Gam_t - Gam_s) (s <= t) is formed from sums over 16-row blocks:
    //   same block:    exp(pi_t - pi_s), pi the prefix sum from the block start,
    //                  summed over the channels on the VALU (exact pairs);
    //   t in block a, s in block b < a:
    //                  exp(pi_t) * exp(sum of the blocks between) * exp(tau_b - pi_s),
    //                  tau_b the block total, so both MFMA operands carry
    //                  factors <= 1 and the middle one scales one operand.
    // Log-decays are floored at -G_FLOOR so that the sums stay finite.  The
    // state phase is unchanged: K+ and Q+ carry exp(Gam_t), K-^T carries
    // exp(Gam_end - Gam_s), and the per-channel factors on the state side are
    // exp(Gam_end) and 1.
    //
    // LP1: floored log-decays reloaded (16 rows of one channel per thread),
    // block prefix sums to gq (registers), to the fp32 plane pi in the K-
    // region (free: the raw rows are consumed) and block totals to gtot;
    // LP2: diagonal blocks of Diag(b) M (fp32, to ld) and of P (planes);
    // LP3: block-relative K+, Q+ and K- planes, the full K- column in km.
    auto local_planes = [&](float (&gq)[16], float (&km)[16]) {
        float* const pi_f = reinterpret_cast<float*>(reg2);     // [CH][FP]
        {
            const int tp = opq(tid);
            const int cgp = tp % DK, qqp = tp / DK;
            const auto rg = make_rsrc(p.g + (tc0 * H + h) * DK, static_cast<uint32_t>(((n - 1) * H + 1) * DK * 4));
            const uint32_t gv = static_cast<uint32_t>((16 * qqp * H * DK + cgp) * 4);
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                float gr = buf_ldf(rg, gv + static_cast<uint32_t>(r * H * DK * 4), 0);
                gr = gr < -G_FLOOR ? -G_FLOOR : gr;        // NaN stays NaN
                acc += gr;
                gq[r] = acc;
                pi_f[(16 * qqp + r) * FP + cgp] = acc;
            }
            gtot_s[qqp][cgp] = acc;
        }
        __syncthreads();
        {
            // lanes: P2 per (block a, row pair pr), 8 channels each; a lane
            // takes rows pr and 15 - pr of block a (17 pairs (t, s) in all)
            const int tp = opq(tid);
            constexpr int P2 = DK / 8;
            const int part = tp % P2, pr = (tp / P2) % 8, a = tp / (8 * P2);
            const int c0 = 8 * part;
            uint16_t* const plo = kOutHi ? nullptr : pp_l;
            for (int half = 0; half < 2; half++) {
                const int rl = half == 0 ? pr : 15 - pr;
                const int R = 16 * a + rl;
                float kr[8], qr[8], pr8[8];
#pragma unroll
                for (int e = 0; e < 8; e += 4) {
                    *reinterpret_cast<float4*>(kr + e) = *reinterpret_cast<const float4*>(ak_f + R * FP + c0 + e);
                    if constexpr (OUT) *reinterpret_cast<float4*>(qr + e) = *reinterpret_cast<const float4*>(aq_f + R * FP + c0 + e);
                    else *reinterpret_cast<float4*>(qr + e) = float4{0.f, 0.f, 0.f, 0.f};
                    *reinterpret_cast<float4*>(pr8 + e) = *reinterpret_cast<const float4*>(pi_f + R * FP + c0 + e);
                }
                const float sk = rk_s[R], sq = rq_s[R], bt = beta_s[R];
                for (int sl = 0; sl <= rl; sl++) {
                    const int S2 = 16 * a + sl;
                    float ks[8], ps[8];
#pragma unroll
                    for (int e = 0; e < 8; e += 4) {
                        *reinterpret_cast<float4*>(ks + e) = *reinterpret_cast<const float4*>(ak_f + S2 * FP + c0 + e);
                        *reinterpret_cast<float4*>(ps + e) = *reinterpret_cast<const float4*>(pi_f + S2 * FP + c0 + e);
                    }
                    float m = 0.f, pp = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const float w = ks[e] * __expf(pr8[e] - ps[e]);
                        m = fmaf(kr[e], w, m);
                        pp = fmaf(qr[e], w, pp);
                    }
                    m = dpp_group_sum<P2>(m);
                    if constexpr (OUT) pp = dpp_group_sum<P2>(pp);
                    if (part == 0) {
                        const float kn = rk_s[S2];
                        ld_s[a][rl][sl] = sl < rl ? bt * (m * sk * kn) : 0.f;
                        if constexpr (OUT) st_split1(pp_h, plo, R * QS + pcol(S2), pp * sq * kn);
                    }
                }
            }
            // entries above the diagonal of the diagonal blocks: 15 per row pair
            for (int e = part; e < 15; e += P2) {
                const bool first = e < 15 - pr;
                const int rl = first ? pr : 15 - pr;
                const int sl = first ? pr + 1 + e : 1 + e;
                ld_s[a][rl][sl] = 0.f;
                if constexpr (OUT) st_split1(pp_h, plo, (16 * a + rl) * QS + pcol(16 * a + sl), 0.f);
            }
        }
        __syncthreads();
        {
            const int tp = opq(tid);
            const int cgp = tp % DK, qqp = tp / DK;
            const float tau = gq[15];
            float suf = 0.f;                               // blocks after this one
            for (int q2 = qqp + 1; q2 < 4; q2++) suf += gtot_s[q2][cgp];
            float kp[16], qp[16], kb[16];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int t = 16 * qqp + r;
                const float kh = ak_f[t * FP + cgp] * rk_s[t];
                const float qh = OUT ? aq_f[t * FP + cgp] * rq_s[t] : 0.f;
                const float E = __expf(gq[r]);
                const float sl = tau - gq[r];
                kp[r] = kh * E;
                qp[r] = qh * E;
                kb[r] = kh * __expf(sl);
                km[r] = kh * __expf(sl + suf);
            }
            if (qqp == 0) {
                eGr_s[cgp] = 1.f;
                eGCr_s[cgp] = 1.f;
                eGC_s[cgp] = __expf(((gtot_s[0][cgp] + gtot_s[1][cgp]) + gtot_s[2][cgp]) + gtot_s[3][cgp]);
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int idx = (16 * qqp + r) * PS + pcol(cgp);
                st_split2(kp_h, kp_l, idx, PS, kp[r], kp[r + 1]);
                if constexpr (OUT) st_split2(qp_h, qp_l, idx, PS, qp[r], qp[r + 1]);
                st_split2(km_h, km_l, idx, PS, kb[r], kb[r + 1]);
            }
        }
    };
    // LP4 (in place of A5): the off-diagonal blocks (a > b) of L and P from the
    // block-relative planes, blocks two or three apart with the decay of the
    // blocks between them applied to the K- operand; P's upper blocks zeroed.
    auto local_products = [&]() {
        const int tp = opq(tid);
        const int ln = tp & 63, wv5 = __builtin_amdgcn_readfirstlane(tp >> 6), gg = ln >> 4, lc = ln & 15;
        for (int ji = wv5; ji < 16; ji += NW) {
            const int job = static_cast<int>((kA5Order >> (4 * ji)) & 15);
            const int a = job >> 2, b = job & 3;
            if (a == b) continue;
            if (a < b) {
                if constexpr (OUT) {
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int idx = (16 * a + 4 * gg + e) * QS + pcol(16 * b + lc);
                        pp_h[idx] = 0;
                        if constexpr (!kOutHi) pp_l[idx] = 0;
                    }
                }
                continue;
            }
            f32x4 am = {0.f, 0.f, 0.f, 0.f}, ap = am;
            for (int ks = 0; ks < KS; ks++) {
                const int offa = (16 * a + lc) * PS + 32 * ks + 8 * gg;
                Frag fb = ld_nat(km_h, km_l, (16 * b + lc) * PS + 32 * ks + 8 * gg);
                if (a >= b + 2) {
                    float d[8];
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        const int c = 32 * ks + 16 * (e >> 2) + 4 * gg + (e & 3);   // channel at 8 gg + e (pcol order)
                        float s2 = gtot_s[b + 1][c];
                        if (a == b + 3) s2 += gtot_s[b + 2][c];
                        d[e] = __expf(s2);
                    }
                    fb = scale_frag(fb, d);
                }
                am = mfma3(ld_nat(kp_h, kp_l, offa), fb, am);
                if constexpr (OUT) ap = mfma3(ld_nat(qp_h, qp_l, offa), fb, ap);
            }
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                const int t = 16 * a + 4 * gg + e, s2 = 16 * b + lc, s2p = pcol(s2);
                if constexpr (OUT && kOutHi) {
                    const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{ap[e], ap[e + 1]}, bf16x2));
                    pp_h[t * QS + s2p] = static_cast<uint16_t>(hw);
                    pp_h[(t + 1) * QS + s2p] = static_cast<uint16_t>(hw >> 16);
                } else if constexpr (OUT) {
                    st_split2(pp_h, pp_l, t * QS + s2p, QS, ap[e], ap[e + 1]);
                }
                st_split2(lp_h, lp_l, t * QS + s2, QS, beta_s[t] * am[e], beta_s[t + 1] * am[e + 1]);
            }
        }
    };
    // LP5 (beside A6): K+ and Q+ planes from block-relative to chunk factors,
    // exp(pi_t) * exp(sum of the earlier blocks) = exp(Gam_t).
    auto local_rescale = [&]() {
        const int tp = opq(tid);
        const int cgp = tp % DK, qqp = tp / DK;
        float pre = 0.f;
        for (int q2 = 0; q2 < qqp; q2++) pre += gtot_s[q2][cgp];
        const float E = __expf(pre);
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int idx = (16 * qqp + r) * PS + pcol(cgp);
            st_split1(kp_h, kp_l, idx, ld_pair(kp_h, kp_l, idx) * E);
            if constexpr (OUT) st_split1(qp_h, qp_l, idx, ld_pair(qp_h, qp_l, idx) * E);
        }
    };

    while (done < L) {
        float vh[4][4];    // SiLU(conv(v)) in accumulator layout
        float km[16];      // K- column of this thread, kept for the transposed copy
        float (&gq)[16] = stg.gq;   // log decay of this thread's (channel, quarter), then its prefix sums
        int n_next_p = 0;           // producer: length of the next chunk
        char* const rslot = ROLE == FUSED ? nullptr : ring + (chunk % RING) * pair_slot_bytes<D, ACT>();

        if constexpr (ROLE != CONSUMER) {

        // ---------------- A2: causal conv + SiLU (q, k channels to LDS; v to registers)
        {
            const int tp = opq(tid);
            const int cqk = tp % (2 * DK), half = tp / (2 * DK);
            const int r0 = 32 * half;
            float w0 = A::ld(raw + (r0 + 0) * CR + cqk);
            float w1 = A::ld(raw + (r0 + 1) * CR + cqk);
            float w2 = A::ld(raw + (r0 + 2) * CR + cqk);
            float* dst = cqk < DK ? aq_f + cqk : ak_f + (cqk - DK);
            // the transition pass needs no q
#pragma unroll 4
            for (int t = r0; t < ((OUT || cqk >= DK) ? r0 + 32 : r0); t++) {
                const float w3 = A::ld(raw + (t + 3) * CR + cqk);
                if constexpr (CD) {
                    dst[t * FP] = t < n ? w3 : 0.f;          // the activation itself
                    continue;
                }
                float y = wqk.x * w0;
                y = fmaf(wqk.y, w1, y);
                y = fmaf(wqk.z, w2, y);
                y = fmaf(wqk.w, w3, y);
                dst[t * FP] = t < n ? silu(y) : 0.f;
                w0 = w1;
                w1 = w2;
                w2 = w3;
            }
            const int ln = tp & 63, jc = 16 * (tp >> 6) + (ln & 15), gg = ln >> 4;
#pragma unroll
            for (int tb = 0; tb < 4; tb++) {
                if constexpr (ROLE == PRODUCER) break;       // the consumer convolves v itself
                const int rb = 16 * tb + 4 * gg;
                float x[7];
#pragma unroll
                for (int m = 0; m < 7; m++) x[m] = A::ld(raw + (rb + m) * CR + 2 * DK + jc);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float y = conv4(wv, x[e], x[e + 1], x[e + 2], x[e + 3]);
                    vh[tb][e] = (rb + e) < n ? (CD ? x[e + 3] : silu(y)) : 0.f;
                    if constexpr (!OUT) vst[(4 * tb + e) * NT + tp] = vh[tb][e];
                }
            }
        }
        __syncthreads();

        // ---------------- A3: L2 norms; decay prefix sums within each quarter
        {
            const int tp = opq(tid);
            constexpr int PPT = NT / (2 * CH);          // threads per (row, tensor)
            constexpr int SPAN = DK / PPT;
            const int pair = tp / PPT, part = tp % PPT;
            const int t = pair % CH;
            const float* src = (pair < CH ? aq_f : ak_f) + t * FP + part * SPAN;
            if (OUT || pair >= CH) {      // whole waves: the transition pass needs no q
                float ssum = 0.f;
#pragma unroll
                for (int c = 0; c < SPAN; c += 4) {
                    const float4 a4 = *reinterpret_cast<const float4*>(src + c);
                    ssum = fmaf(a4.x, a4.x, ssum);
                    ssum = fmaf(a4.y, a4.y, ssum);
                    ssum = fmaf(a4.z, a4.z, ssum);
                    ssum = fmaf(a4.w, a4.w, ssum);
                }
                ssum = dpp_group_sum<PPT>(ssum);
                if (part == 0) (pair < CH ? rq_s : rk_s)[t] = rsqrtf(ssum + p.l2_eps);
            }
#pragma unroll
            for (int r = 1; r < 16; r++) gq[r] += gq[r - 1];
            gtot_s[tp / DK][tp % DK] = gq[15];
            // a 16-row block total at or below -FAST_BOUND / 2 (or NaN) sends
            // the chunk to the block-local path
            if (!(gq[15] > -0.5f * FAST_BOUND)) sm.local = 1;
        }
        __syncthreads();
        const int local = __builtin_amdgcn_readfirstlane(sm.local);
        // producer, after the planes are stored: the previous chunk's ring
        // stores were issued a phase ago; once every thread has seen its own
        // complete (no other global access is in flight: this chunk's inputs
        // were committed before phase A), that chunk is published.  Then the
        // next chunk's inputs are requested (the staging registers are free
        // here), so they arrive during A5, A6 and the ring stores.
        auto after_planes = [&]() {
            if constexpr (ROLE == PRODUCER) __builtin_amdgcn_s_waitcnt(VMCNT0);
            __syncthreads();
            if constexpr (ROLE == PRODUCER) {
                if (tid == 0) {
                    if (chunk > 0) __hip_atomic_store(ready_ctr, chunk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    seen = ring_peek(taken_ctr);       // used after A6
                }
                const int done_next = done + n;
                n_next_p = done_next < L ? min(L - done_next, CH - static_cast<int>((pos + n) % CH)) : 0;
                // the raw rows now, the gates before A6: requested together they
                // stall the issue for want of room among the misses in flight
                if (n_next_p > 0) stage_issue<ACT, DK, DV, NT, NTEN, true, false>(stg, p, x0_s, ctx0, tok0 + done_next, n_next_p, H, h, opq(tid));
                else stage_clear(stg);
            }
        };
        if (__builtin_expect(local, 0)) {
            local_planes(gq, km);
            after_planes();
            local_products();
            __syncthreads();
            local_rescale();
        } else {

        // ---------------- A4: K+, K-, Q+ (hi/lo planes); per-channel factors
        {
            const int tp = opq(tid);
            const int cgp = tp % DK, qqp = tp / DK;
            const float t0 = gtot_s[0][cgp], t1 = gtot_s[1][cgp], t2 = gtot_s[2][cgp], t3 = gtot_s[3][cgp];
            const float gam_r = t0 + t1;                  // Gam at the reference row
            const float gam_c = gam_r + t2 + t3;          // Gam at the chunk's last row
            const float off = qqp == 0 ? 0.f : (qqp == 1 ? t0 : (qqp == 2 ? gam_r : gam_r + t2));
            float kp[16], qp[16];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int t = 16 * qqp + r;
                const float d = (gq[r] + off) - gam_r;
                const float E = __expf(d), Ei = __expf(-d);
                const float kh = ak_f[t * FP + cgp] * rk_s[t];
                const float qh = OUT ? aq_f[t * FP + cgp] * rq_s[t] : 0.f;
                kp[r] = kh * E;
                km[r] = kh * Ei;
                qp[r] = qh * E;
            }
            if (qqp == 0) {
                eGr_s[cgp] = __expf(gam_r);
                eGCr_s[cgp] = __expf(gam_c - gam_r);
                eGC_s[cgp] = __expf(gam_c);
            }
            __syncthreads();
            const bool odd = cgp & 1;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int idx = (16 * qqp + r) * PS + pcol(cgp);
                st_split2_x2(kp_h, kp_l, idx, PS, kp[r], kp[r + 1], odd);
                if constexpr (OUT) st_split2_x2(qp_h, qp_l, idx, PS, qp[r], qp[r + 1], odd);
                st_split2_x2(km_h, km_l, idx, PS, km[r], km[r + 1], odd);
            }
        }
        after_planes();

        // ---------------- A5: L = Diag(b) strictLower(K+ K-^T), P = lower(Q+ K-^T);
        // one job per 16x16 block pair (a, b) computes both, sharing the K-
        // fragments.  Only the 10 jobs with a >= b multiply; wave w takes jobs
        // kA5Order[w + i NW], an order that gives the SIMDs 3, 3, 2 and 2 of them
        // with 8 waves (waves w and w + 4 share a SIMD), 3, 3, 2, 2 with 4 and
        // 5, 5 with 2.
        {
            const int tp = opq(tid);
            const int ln = tp & 63, wv5 = __builtin_amdgcn_readfirstlane(tp >> 6), gg = ln >> 4, lc = ln & 15;
            for (int ji = wv5; ji < 16; ji += NW) {
                const int job = static_cast<int>((kA5Order >> (4 * ji)) & 15);
                const int a = job >> 2, b = job & 3;
                if (a < b) {
                    if constexpr (OUT) {
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const int idx = (16 * a + 4 * gg + e) * QS + pcol(16 * b + lc);
                            pp_h[idx] = 0;
                            if constexpr (!kOutHi) pp_l[idx] = 0;   // with bf16 outputs only P's hi plane is read
                        }
                    }
                    continue;
                }
                f32x4 am = {0.f, 0.f, 0.f, 0.f}, ap = am;
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    const int offa = (16 * a + lc) * PS + 32 * ks + 8 * gg;
                    const Frag fb = ld_nat(km_h, km_l, (16 * b + lc) * PS + 32 * ks + 8 * gg);
                    am = mfma3(ld_nat(kp_h, kp_l, offa), fb, am);
                    if constexpr (OUT) ap = mfma3(ld_nat(qp_h, qp_l, offa), fb, ap);
                }
#pragma unroll
                for (int e = 0; e < 4; e += 2) {
                    const int t = 16 * a + 4 * gg + e, s2 = 16 * b + lc, s2p = pcol(s2);
                    if constexpr (OUT && kOutHi) {
                        // hi plane only (the same rounding as split2's hi)
                        const uint32_t hw = __builtin_bit_cast(
                            uint32_t, __builtin_convertvector(f32x2{t >= s2 ? ap[e] : 0.f, t + 1 >= s2 ? ap[e + 1] : 0.f},
                                                              bf16x2));
                        pp_h[t * QS + s2p] = static_cast<uint16_t>(hw);
                        pp_h[(t + 1) * QS + s2p] = static_cast<uint16_t>(hw >> 16);
                    } else if constexpr (OUT) {
                        st_split2(pp_h, pp_l, t * QS + s2p, QS, t >= s2 ? ap[e] : 0.f, t + 1 >= s2 ? ap[e + 1] : 0.f);
                    }
                    if (a > b) {
                        st_split2(lp_h, lp_l, t * QS + s2, QS, beta_s[t] * am[e], beta_s[t + 1] * am[e + 1]);
                    } else {
                        ld_s[a][4 * gg + e][lc] = t > s2 ? beta_s[t] * am[e] : 0.f;
                        ld_s[a][4 * gg + e + 1][lc] = t + 1 > s2 ? beta_s[t + 1] * am[e + 1] : 0.f;
                    }
                }
            }
        }
        __syncthreads();
        }   // fast path of A4 and A5

        // ---------------- A6: T_aa = (I + L_aa)^{-1} for the 4 diagonal blocks,
        // forward substitution on one column with PARTS threads splitting each
        // dot product; then the K-^T planes into the K- region
        {
            const int tp = opq(tid);
            if (tp == 0) sm.local = 0;                   // read after A3: free for the next chunk
            // the next chunk's log-decays and beta (its raw rows follow A4 in a
            // producer, phase B in one workgroup per chain)
            if constexpr (ROLE == PRODUCER) {
                if (n_next_p > 0)
                    stage_issue<ACT, DK, DV, NT, NTEN, false, true>(stg, p, x0_s, ctx0, tok0 + done + n, n_next_p, H, h, tp);
            } else if constexpr (ROLE == FUSED) {
                const int dn = done + n;
                const int nn = dn < L ? min(L - dn, CH - static_cast<int>((pos + n) % CH)) : 0;
                if (nn > 0) stage_issue<ACT, DK, DV, NT, NTEN, false, true>(stg, p, x0_s, ctx0, tok0 + dn, nn, H, h, tp);
            }
            constexpr int PARTS = NT / 64, KPP = 16 / PARTS;
            const int part = tp % PARTS, col = (tp / PARTS) % 16, blk = tp / (16 * PARTS);
            float xk[KPP];
#pragma unroll
            for (int kk = 0; kk < KPP; kk++) xk[kk] = 0.f;
            // this thread's entries of the block, all requested before the
            // substitution so that its 16 dependent steps do not each wait for LDS
            float lb[16][KPP];
#pragma unroll
            for (int r = 0; r < 16; r++)
#pragma unroll
                for (int kk = 0; kk < KPP; kk++) lb[r][kk] = ld_s[blk][r][part * KPP + kk];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                float c2 = 0.f;
#pragma unroll
                for (int kk = 0; kk < KPP; kk++) c2 = fmaf(lb[r][kk], xk[kk], c2);
                const float sdot = dpp_group_sum<PARTS>(c2);
                const float xr = r < col ? 0.f : (r == col ? 1.f : -sdot);
#pragma unroll
                for (int kk = 0; kk < KPP; kk++)
                    if (part * KPP + kk == r) xk[kk] = xr;
            }
#pragma unroll
            for (int kk = 0; kk < KPP; kk += 2)
                st_split2(lp_h, lp_l, (16 * blk + part * KPP + kk) * QS + 16 * blk + col, QS, xk[kk], xk[kk + 1]);
            const int cgp = tp % DK, qqp = tp / DK;
            st_kt<QS>(kt_h, kt_l, cgp, qqp, km);
        }
        __syncthreads();
        }   // phase A

        const auto rr = make_rsrc(rslot, static_cast<uint32_t>(pair_slot_bytes<D, ACT>()));
        if constexpr (ROLE == PRODUCER) {
            // hand the chunk over: wait until the consumer has taken the
            // chunk that last used this slot, then store planes and sv
            // (published in the next chunk's phase A, or after the last
            // chunk)
            if (chunk >= RING) {
                if (tid == 0) sm.flag = ring_wait(taken_ctr, chunk - RING + 1, seen, p.spin_limit, p.status);
                __syncthreads();
                if (!sm.flag) return;                         // the consumer is gone
            }
            const int done_next = done + n;
            const int64_t pos_next = pos + n;
            const int n_next = n_next_p;
            {
                const int tp = opq(tid);
                ring_put<NPA, NT, 6>(rr, 0, reinterpret_cast<const uint4*>(lds), tp);
                ring_put<NPB, NT, 6>(rr, PB0, reinterpret_cast<const uint4*>(lds) + PB0, tp);
                if (tp < NSV) ring_st(rr, NPW + tp, reinterpret_cast<const uint4*>(sm.sv)[tp]);
            }
            // every thread has read its planes, sv and beta out of LDS
            // (its stores need not be complete) before the next chunk's raw
            // rows and beta overwrite them
            __syncthreads();
            if (n_next > 0) stage_commit<ACT, DK, DV, NT, NTEN>(stg, raw, beta_s, opq(tid));
            done = done_next;
            pos = pos_next;
            n = n_next;
            tc0 = tok0 + done;
            chunk++;
            __syncthreads();
            continue;
        }
        if constexpr (ROLE == CONSUMER) {
            // take the chunk over: the chunk's raw v rows (with 3 rows of
            // left context) were requested into vwin during the previous
            // chunk's epilogue (the first chunk's here); wait for the chunk,
            // then planes and sv into LDS
            if (chunk == 0) vwin_copy<ACT, DV, NW>(p, vwin, ctx0, tc0, n, H, h, wave, lane);
            const bool early = sm.early;
            if (!early) {
            if (tid == 0) sm.flag = ring_wait(ready_ctr, chunk + 1, seen, p.spin_limit, p.status);
            __syncthreads();
            }
            if (!early && !sm.flag) {
                // the producer is gone: NaN outputs from here on, and NaN in
                // this head's state of every checkpoint still due and of the
                // final slot, so that none of them passes for a valid state
                // (the v-row copy into LDS lands before the workgroup ends)
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                for (int64_t e = tid; e < static_cast<int64_t>(L - done) * DV; e += NT) {
                    const int64_t t = tc0 + e / DV;
                    A::st(out + (t * H + h) * DV + e % DV, nan_f32());
                }
                auto nan_state = [&](void* pool, int64_t slot) {
                    const int64_t sh = (slot * H + h) * DK * DV;
                    for (int e = tid; e < DK * DV; e += NT) {
                        if (p.state_bf16) static_cast<uint16_t*>(pool)[sh + e] = 0x7fc0u;
                        else static_cast<float*>(pool)[sh + e] = nan_f32();
                    }
                };
                if (p.ckpt_interval > 0) {
                    const int64_t I = p.ckpt_interval;
                    const int64_t total = (start + L - 1) / I - start / I + 1;   // checkpoints of the sequence
                    for (int64_t j = ck; j < total; j++) {
                        const int64_t slot = ck_base + j;
                        if (slot >= 0 && slot < p.num_ckpt_slots) nan_state(p.ckpt_state, slot);
                    }
                }
                if (fin >= 0 && fin < p.num_slots) nan_state(p.state, fin);
                return;
            }
            {
                const int tp = opq(tid);
                if (!early) {
                    ring_get2<NPA, PB0, NPB, NT>(rr, reinterpret_cast<uint4*>(lds), tp);
                    if (tp < NSV) reinterpret_cast<uint4*>(sm.sv)[tp] = ring_ld(rr, NPW + tp);
                }
                // this wave's copies into LDS (the v rows, and with an early
                // take-over the slot, issued after the previous chunk's phase B)
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                vwin_fix<ACT, DK, DV, NT>(vwin, x0_s, ctx0, tc0, tp);
            }
            __syncthreads();
            {
                // SiLU(conv(v)) in accumulator layout, as phase A computes it
                const int tp = opq(tid);
                const int ln = tp & 63, jc = 16 * (tp >> 6) + (ln & 15), gg = ln >> 4;
#pragma unroll
                for (int tb = 0; tb < 4; tb++) {
                    const int rb = 16 * tb + 4 * gg;
                    float x[7];
#pragma unroll
                    for (int m = 0; m < 7; m++) x[m] = A::ld(vwin + (rb + m) * DV + jc);
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float y = conv4(wv, x[e], x[e + 1], x[e + 2], x[e + 3]);
                        vh[tb][e] = (rb + e) < n ? (CD ? x[e + 3] : silu(y)) : 0.f;
                    }
                }
            }
        }

        // consumer: a fresh look at the producer's counter, returned during
        // phase B, decides whether the next slot is requested right after it
        if (ROLE == CONSUMER && tid == 0) seen = ring_peek(ready_ctr);

        // ---------------- B: state-dependent part; wave = 16-column strip of S
        f32x4 accr[4];     // readouts O (rows 16tb + 4g + e, this lane's column)
        float zr[4][4];    // output gate inputs, requested before the MFMA work
        const uint32_t rowb = static_cast<uint32_t>(H * DV * sizeof(ACT));
        const uint32_t nb = static_cast<uint32_t>(((n - 1) * H + 1) * DV * sizeof(ACT));
        {
            const int tp = opq(tid);
            const int ln = tp & 63, gg = ln >> 4, lc = ln & 15;
            if constexpr (OUT) {
                // rows past the chunk fall outside the resource (range-checked
                // per-lane offsets) and read as zero
                const auto rz = make_rsrc(zin + (tc0 * H + h) * DV, nb);
                const uint32_t vo = static_cast<uint32_t>(4 * gg * rowb + (16 * (tp >> 6) + lc) * sizeof(ACT));
#pragma unroll
                for (int tb = 0; tb < 4; tb++)
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        zr[tb][e] = buf_ld_act<ACT>(rz, vo + static_cast<uint32_t>((16 * tb + e) * rowb), 0);
            }
            // one state strip through the chunk: S (or, for the transition pass's F, the
            // strip propagated from the identity, with v taken as zero)
            auto state_step = [&](f32x4 (&Sx)[IB], bool zero_v, int o) {
                // the LDS operands at offset o (elements): an offset the optimiser cannot
                // see keeps the second strip's loads from being merged with the first's,
                // whose values would otherwise stay in registers across both strips
                const float* const eGr_s_o = eGr_s + o;
                const float* const beta_s_o = beta_s + o;
                const float* const eGC_s_o = eGC_s + o;
                const float* const eGCr_s_o = eGCr_s + o;
                const uint16_t* const kp_h_o = kp_h + o;
                const uint16_t* const kp_l_o = kp_l + o;
                const uint16_t* const qp_h_o = qp_h + o;
                const uint16_t* const qp_l_o = qp_l + o;
                const uint16_t* const lp_h_o = lp_h + o;
                const uint16_t* const lp_l_o = lp_l + o;
                const uint16_t* const pp_h_o = pp_h + o;
                const uint16_t* const pp_l_o = pp_l + o;
                const uint16_t* const kt_h_o = kt_h + o;
                const uint16_t* const kt_l_o = kt_l + o;
                const float* const vst_o = vst + o;
                f32x4 accx[4];
#pragma unroll
                for (int tb = 0; tb < 4; tb++) {
                    accx[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
                    accr[tb] = accx[tb];
                }
                // K_g S and Q_g S: the per-channel exp(Gam_r) goes onto S's rows.  K+ keeps
                // about fp32 accuracy; with bf16 outputs Q+ (outputs only) is rounded once
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        x[e] = eGr_s_o[32 * ks + 4 * gg + e] * Sx[2 * ks][e];
                        x[e + 4] = eGr_s_o[32 * ks + 16 + 4 * gg + e] * Sx[2 * ks + 1][e];
                    }
                    const Frag fs = split8(x);
#pragma unroll
                    for (int tb = 0; tb < 4; tb++) {
                        const int off = (16 * tb + lc) * PS + 32 * ks + 8 * gg;
                        accx[tb] = mfma3(ld_nat(kp_h_o, kp_l_o, off), fs, accx[tb]);
                        if constexpr (!OUT) continue;
                        if constexpr (kOutHi) accr[tb] = mfma2(ld_nat_hi(qp_h_o, off), fs, accr[tb]);
                        else accr[tb] = mfma3(ld_nat(qp_h_o, qp_l_o, off), fs, accr[tb]);
                    }
                }
                // Y = Diag(b) (V - K_g S)
                f32x4 y[4];
#pragma unroll
                for (int tb = 0; tb < 4; tb++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float v = zero_v ? 0.f : (OUT ? vh[tb][e] : vst_o[(4 * tb + e) * NT + tp]);
                        y[tb][e] = beta_s_o[16 * tb + 4 * gg + e] * (v - accx[tb][e]);
                    }
                // U: solve (I + L) U = Y block by block, U_a = T_aa (Y_a - sum_{c<a} L_ac U_c)
                Frag4 fu[4];
#pragma unroll
                for (int a = 0; a < 4; a++) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c2 = 0; c2 < a; c2++)
                        acc = mfma3_16(ld4(lp_h_o, lp_l_o, (16 * a + lc) * QS + 16 * c2 + 4 * gg), fu[c2], acc);
                    f32x4 r;
#pragma unroll
                    for (int e = 0; e < 4; e++) r[e] = y[a][e] - acc[e];
                    const f32x4 ua = mfma3_16(ld4(lp_h_o, lp_l_o, (16 * a + lc) * QS + 16 * a + 4 * gg), split4(r),
                                              f32x4{0.f, 0.f, 0.f, 0.f});
                    fu[a] = split4(ua);
                }
                const Frag fu0 = cat(fu[0], fu[1]);
                const Frag fu1 = cat(fu[2], fu[3]);
                // O = Q_g S + P U (with bf16 outputs, Q+ and P are rounded once to bf16)
#pragma unroll
                for (int tb = 0; tb < 4; tb++) {
                    if constexpr (!OUT) break;
                    const int row = (16 * tb + lc) * QS + 8 * gg;
                    if constexpr (kOutHi) {
                        accr[tb] = mfma2(ld_nat_hi(pp_h_o, row), fu0, accr[tb]);
                        if (tb >= 2) accr[tb] = mfma2(ld_nat_hi(pp_h_o, row + 32), fu1, accr[tb]);
                    } else {
                        accr[tb] = mfma3(ld_nat(pp_h_o, pp_l_o, row), fu0, accr[tb]);
                        if (tb >= 2) accr[tb] = mfma3(ld_nat(pp_h_o, pp_l_o, row + 32), fu1, accr[tb]);
                    }
                }
                // S = Diag(exp Gam_end) S + Diag(exp(Gam_end - Gam_r)) K-^T U
#pragma unroll
                for (int ib = 0; ib < IB; ib++) {
                    const int row = (16 * ib + lc) * QS + 8 * gg;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                    acc = mfma3(ld_nat(kt_h_o, kt_l_o, row), fu0, acc);
                    acc = mfma3(ld_nat(kt_h_o, kt_l_o, row + 32), fu1, acc);
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int i = 16 * ib + 4 * gg + e;
                        Sx[ib][e] = fmaf(eGC_s_o[i], Sx[ib][e], eGCr_s_o[i] * acc[e]);
                    }
                }
            };
            state_step(S, false, 0);
            if constexpr (!OUT) {
                // F's strip after G's: every G value is final before F's operands
                // are requested (asm statements keep their order)
#pragma unroll
                for (int ib = 0; ib < IB; ib++) asm volatile("" : "+v"(S[ib]));
                state_step(SF, true, opq(0));
            }
            // row sums of O^2 over this wave's 16 columns
            if constexpr (OUT) {
#pragma unroll
                for (int tb = 0; tb < 4; tb++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float s2 = dpp_group_sum<16>(accr[tb][e] * accr[tb][e]);
                        if (lc == 0) part_s[tp >> 6][16 * tb + 4 * gg + e] = s2;
                    }
            }
        }
        const int done_next = done + n;
        const int64_t pos_next = pos + n;
        const int n_next = done_next < L ? min(L - done_next, CH - static_cast<int>(pos_next % CH)) : 0;
        // consumer: when the next chunk was already published at the last
        // look at its counter, its slot is requested now, straight into the
        // planes (free once phase B is done), and lands during the epilogue
        if (ROLE == CONSUMER && tid == 0) sm.early = n_next > 0 && seen >= chunk + 2;
        __syncthreads();

        if constexpr (ROLE == CONSUMER) {
            if (sm.early) {
                ring_get2_async<NPA, PB0, NPB, NSV, NPW, NW>(
                    ring + ((chunk + 1) % RING) * pair_slot_bytes<D, ACT>(),
                    static_cast<uint32_t>(pair_slot_bytes<D, ACT>()), lds, sm.sv, wave, lane);
            }
            // the next chunk's v rows (vwin was last read before phase B)
            if (n_next > 0) vwin_copy<ACT, DV, NW>(p, vwin, ctx0, tok0 + done_next, n_next, H, h, wave, lane);
        }

        // ---------------- next chunk's inputs: loads in flight during the epilogue
        if constexpr (ROLE == FUSED) {
            if (n_next > 0) stage_issue<ACT, DK, DV, NT, NTEN, true, false>(stg, p, x0_s, ctx0, tok0 + done_next, n_next, H, h, opq(tid));
            else stage_clear(stg);
        } else {
            // every read of this slot is complete (its values fed phase B):
            // the producer may refill it
            if (tid == 0) {
                __hip_atomic_store(taken_ctr, chunk + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                seen = ring_peek(ready_ctr);       // used at the next chunk's take-over
            }
        }

        // ---------------- epilogue: gated RMSNorm over dv, then the outputs
        if constexpr (OUT) {
        if (tid < CH) {
            float tot = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; w2++) tot += part_s[w2][tid];
            rinv_s[tid] = rsqrtf(tot * (1.0f / DV) + p.rms_eps);
        }
        __syncthreads();
        {
            const int tp = opq(tid);
            const int ln = tp & 63, gg = ln >> 4, jc = 16 * (tp >> 6) + (ln & 15);
            const auto ro = make_rsrc(out + (tc0 * H + h) * DV, nb);
            const uint32_t vo = static_cast<uint32_t>(4 * gg * rowb + jc * sizeof(ACT));
#pragma unroll
            for (int tb = 0; tb < 4; tb++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int t = 16 * tb + 4 * gg + e;
                    const float rinv = rinv_s[t];
                    // rows past the chunk lie outside the resource (the row offset is
                    // in the range-checked per-lane offset): those stores are dropped
                    buf_st_act<ACT>(ro, vo + static_cast<uint32_t>((16 * tb + e) * rowb), 0,
                                    accr[tb][e] * rinv * nwj * sigmoid(zr[tb][e]));
                }
        }
        }

        // the raw-row region and beta are free: every wave is past its state phase
        if (ROLE == FUSED && n_next > 0) stage_commit<ACT, DK, DV, NT, NTEN>(stg, raw, beta_s, opq(tid));
        done = done_next;
        pos = pos_next;
        // ---------------- checkpoints: interval boundaries inside, and the end
        if (OUT && p.ckpt_interval > 0 && (pos % p.ckpt_interval == 0 || done == L)) {
            const int slot = ck_base + ck;
            ck++;
            if (slot >= 0 && slot < p.num_ckpt_slots) {
                const int64_t sh = static_cast<int64_t>(slot) * H + h;
                store_pool_strip<IB, DV>(p.ckpt_state, sh, S, g4, jcol, DK, p.state_bf16);
                write_conv_state(static_cast<ACT*>(p.ckpt_conv) + sh * C * 3, tok0 + done);
            } else if (p.state_bf16) {
                // no slot to write, but the stored dtype still applies here
#pragma unroll
                for (int ib = 0; ib < IB; ib++)
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        S[ib][e] = __uint_as_float(static_cast<uint32_t>(bf16_bits(static_cast<__bf16>(S[ib][e]))) << 16);
            }
        }
        n = n_next;
        tc0 = tok0 + done;
        chunk++;
        __syncthreads();
    }
    if constexpr (ROLE == PRODUCER) {
        // publish the last chunk
        __builtin_amdgcn_s_waitcnt(VMCNT0);
        __syncthreads();
        if (tid == 0 && chunk > 0) __hip_atomic_store(ready_ctr, chunk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }

    if constexpr (OUT) {
        if (fin >= 0 && fin < p.num_slots) {
            const int64_t sh = static_cast<int64_t>(fin) * H + h;
            store_pool_strip<IB, DV>(p.state, sh, S, g4, jcol, DK, p.state_bf16);
            write_conv_state(static_cast<ACT*>(p.conv) + sh * C * 3, tok0 + L);
        }
    } else {
        const int64_t sh = (static_cast<int64_t>(item) * H + h) * DK * DV;
        store_state_strip<IB, DV>(p.seg_G + sh, S, g4, jcol, DK);
        store_state_strip<IB, DV>(p.seg_F + sh, SF, g4, jcol, DK);
    }
}

// One workgroup per chain (OUT), or per segment transition (!OUT: its G and
// F together).
template <int D, typename ACT, bool OUT, bool CD>
__global__ __launch_bounds__(4 * D) void prefill_kernel(PrefillParams p) {
    __shared__ PrefillLds<D, ACT> sm;
    const int b = static_cast<int>(blockIdx.x);
    prefill_chain<D, ACT, OUT, FUSED, CD>(p, sm, b / p.H, b % p.H);
}

// A resident grid of G workgroups, launched cooperatively so that all of
// them run at once (a consumer waits on its producer and the other way
// round).  The first K chains in work order (the longest; K chosen by the
// metadata kernel) get two workgroups each: blocks 16m .. 16m+7 produce for
// chains 8m .. 8m+7 and blocks 16m+8 .. 16m+15 consume them, so the two
// workgroups of a chain have block indices equal mod 8, which places them in
// the same L2 when workgroups are dealt round-robin over the 8 XCDs.  Every
// other workgroup, and each pair once its chain is done, takes the remaining
// chains one at a time from a queue, longest first, and runs each in one
// workgroup.
// QUEUE = false: every chain is paired (the grid holds them all), and the
// one-workgroup code is left out of the kernel, which keeps the two roles'
// register allocation free of it.
template <int D, typename ACT, bool QUEUE, bool CD>
__global__ __launch_bounds__(4 * D) void prefill_pair_kernel(PrefillParams p) {
    __shared__ PrefillLds<D, ACT> sm;
    __shared__ int next_s;
    const int NH = p.N * p.H;
    const int32_t* sched = p.ring_ctr + static_cast<int64_t>(p.max_pairs) * 32;
    const int K = sched[0];
    const int b = blockIdx.x;
    const int pair = 8 * (b / 16) + (b % 8);
    if (pair < K) {
        if ((b % 16) < 8) prefill_chain<D, ACT, true, PRODUCER, CD>(p, sm, pair / p.H, pair % p.H);
        else prefill_chain<D, ACT, true, CONSUMER, CD>(p, sm, pair / p.H, pair % p.H);
        __syncthreads();
    }
    if constexpr (!QUEUE) return;
    for (;;) {
        if (threadIdx.x == 0) next_s = atomicAdd(const_cast<int32_t*>(sched) + 1, 1);
        __syncthreads();
        const int chain = K + next_s;
        __syncthreads();
        if (chain >= NH) break;
        prefill_chain<D, ACT, true, FUSED, CD>(p, sm, chain / p.H, chain % p.H);
        __syncthreads();
    }
}

// Chunks of 64 a work item runs (the grid is aligned to absolute positions).
__device__ __forceinline__ int64_t item_chunks(const SeqWork& w) {
    if (w.len <= 0) return 0;
    const int64_t s0 = w.start < 0 ? 0 : w.start % CH;
    return (s0 + w.len + CH - 1) / CH;
}

// Scheduled launch (one workgroup of 1024 threads, after the work items are
// written): zero the ring counters and the chain queue, and choose K, the
// number of leading chains that get a producer/consumer pair.  Cost model in
// chunk steps of one workgroup: a paired chain costs 0.72 per chunk (its two
// halves overlap), a single one 1; the G - 2K unpaired workgroups share the
// other chains.  K minimises the larger of the longest paired chain, the
// longest single chain and the single chains' total over those workgroups.
__device__ void schedule_pairs(const SeqWork* work, int32_t N, int32_t H, int32_t* ring_ctr, int32_t max_pairs,
                               int32_t grid) {
    __shared__ double part_s[1024];
    __shared__ float lead_s[PAIR_MAX_PAIRS + 1];      // chunks of the leading items
    for (int64_t i = threadIdx.x; i < static_cast<int64_t>(max_pairs) * 32 + 32; i += 1024) ring_ctr[i] = 0;
    double tot = 0.0;
    for (int i = threadIdx.x; i < N; i += 1024) {
        const int64_t c = item_chunks(work[i]);
        tot += static_cast<double>(c);
        if (i <= PAIR_MAX_PAIRS) lead_s[i] = static_cast<float>(c);
    }
    part_s[threadIdx.x] = tot;
    __syncthreads();
    for (int off = 512; off > 0; off >>= 1) {
        if (static_cast<int>(threadIdx.x) < off) part_s[threadIdx.x] += part_s[threadIdx.x + off];
        __syncthreads();
    }
    if (threadIdx.x != 0) return;
    const int64_t NH = static_cast<int64_t>(N) * H;
    if (2 * NH <= grid && NH <= max_pairs) {
        // the grid holds a pair for every chain: pair them all
        ring_ctr[static_cast<int64_t>(max_pairs) * 32] = static_cast<int32_t>(NH);
        return;
    }
    const double W = part_s[0] * H;                  // chunk steps of all chains
    const int64_t kmax = min(min(static_cast<int64_t>(max_pairs), static_cast<int64_t>(grid / 2)), NH);
    const double l0 = NH > 0 ? lead_s[0] : 0.0;
    double best = 1e300, paired = 0.0;
    int bestk = 0;
    for (int64_t k = 0; k <= kmax; k++) {
        const double lu = k < NH ? lead_s[k / H] : 0.0;   // k / H <= kmax <= PAIR_MAX_PAIRS
        const int64_t workers = grid - 2 * k;
        if (k == NH || workers > 0) {
            const double rest = W - paired;
            const double mk = fmax(fmax(k > 0 ? 0.72 * l0 : 0.0, lu), workers > 0 ? rest / workers : 0.0);
            if (mk < best * (1.0 - 1e-9)) {
                best = mk;
                bestk = static_cast<int>(k);
            }
        }
        if (k < NH) paired += lu;
    }
    ring_ctr[static_cast<int64_t>(max_pairs) * 32] = bestk;
}

// One workgroup: per-sequence work items ordered longest first, so the
// longest chains start first.  Sequences with bounds outside [0, T] get
// len = -1 and are skipped by the prefill kernel.
__global__ __launch_bounds__(1024) void prefill_meta_kernel(const int32_t* cu, const int64_t* sp, int32_t N,
                                                            int64_t T, SeqWork* work, int32_t H, int32_t* ring_ctr,
                                                            int32_t max_pairs, int32_t grid, int32_t* status) {
    if (threadIdx.x == 0) *status = 0;
    for (int i = threadIdx.x; i < N; i += 1024) {
        const int64_t a = cu[i], b = cu[i + 1];
        const bool ok = a >= 0 && b >= a && b <= T;
        const int32_t li = ok ? static_cast<int32_t>(b - a) : -1;
        int rank = i;
        if (N <= 1024) {
            rank = 0;
            for (int j = 0; j < N; j++) {
                const int64_t aj = cu[j], bj = cu[j + 1];
                const int32_t lj = (aj >= 0 && bj >= aj && bj <= T) ? static_cast<int32_t>(bj - aj) : -1;
                rank += (lj > li) || (lj == li && j < i);
            }
        }
        SeqWork w;
        w.seq = i;
        w.tok0 = ok ? static_cast<int32_t>(a) : 0;
        w.len = li;
        w.ctx0 = w.tok0;
        w.start = sp ? sp[i] : 0;
        w.part = 0;
        w.last = 1;
        work[rank] = w;
    }
    // work[i] was written by the thread that ranked sequence i, not by
    // thread i: every write must be complete before the schedule reads them
    __syncthreads();
    if (ring_ctr) schedule_pairs(work, N, H, ring_ctr, max_pairs, grid);
}

// Segments of sequence i when sequences are cut at the checkpoint positions
// strictly inside (start, start+len); 1 (no cut) for an empty or malformed
// sequence, a negative start or an invalid initial slot.
__device__ int32_t split_count(const PrefillParams& p, int i, int64_t* a_out, int64_t* len_out,
                               int64_t* start_out, int64_t* first_out) {
    const int64_t a = p.cu_seqlens[i], b = p.cu_seqlens[i + 1];
    const bool ok = a >= 0 && b >= a && b <= p.T;
    const int64_t start = p.start_pos ? p.start_pos[i] : 0;
    const int init = p.init_slot ? p.init_slot[i] : -1;
    *a_out = a;
    *len_out = ok ? b - a : -1;
    *start_out = start;
    *first_out = 0;
    if (!ok || b == a || start < 0 || init < -1 || init >= p.num_slots) return 1;
    const int64_t I = p.ckpt_interval;
    const int64_t first = (start / I + 1) * I;        // first checkpoint position after start
    const int64_t endm1 = start + (b - a) - 1;          // cuts at positions <= start+len-1
    *first_out = first;
    return endm1 >= first ? static_cast<int32_t>((endm1 - first) / I + 2) : 1;
}

// One workgroup: items of every sequence in order, segments contiguous.
// Should the segments not fit the allocated items (only possible when the
// sequences overlap), no sequence is cut.
__global__ __launch_bounds__(1024) void prefill_split_meta_kernel(PrefillParams p) {
    __shared__ int32_t scan_s[1024];
    __shared__ int64_t total_s;
    const int tid = threadIdx.x;
    if (tid == 0) {
        total_s = 0;
        *p.status = 0;
    }
    __syncthreads();
    for (int base = 0; base < p.N; base += 1024) {
        const int i = base + tid;
        int64_t a, len, start, first;
        const int32_t ns = i < p.N ? split_count(p, i, &a, &len, &start, &first) : 0;
        scan_s[tid] = ns;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int32_t x = tid >= off ? scan_s[tid - off] : 0;
            __syncthreads();
            scan_s[tid] += x;
            __syncthreads();
        }
        const int64_t first_item = total_s + scan_s[tid] - ns;
        if (i < p.N) p.seq_items[i] = make_int2(static_cast<int>(min(first_item, static_cast<int64_t>(INT32_MAX))), ns);
        __syncthreads();
        if (tid == 1023) total_s += scan_s[1023];
        __syncthreads();
    }
    const bool fits = total_s <= p.max_items;
    // each thread reads back only the entries it wrote itself
    for (int i = tid; i < p.N; i += 1024) {
        int64_t a, len, start, first;
        int32_t ns = split_count(p, i, &a, &len, &start, &first);
        int32_t it0 = p.seq_items[i].x;
        if (!fits) {
            ns = 1;
            it0 = i;
            p.seq_items[i] = make_int2(i, 1);
        }
        for (int m = 0; m < ns; m++) {
            const int64_t I = p.ckpt_interval;
            const int64_t p0 = m == 0 ? start : first + (m - 1) * I;
            const int64_t p1 = m == ns - 1 ? start + len : first + m * I;
            SeqWork w;
            w.seq = i;
            w.tok0 = len >= 0 ? static_cast<int32_t>(a + (p0 - start)) : 0;
            w.len = len >= 0 ? static_cast<int32_t>(p1 - p0) : -1;
            w.ctx0 = len >= 0 ? static_cast<int32_t>(a) : 0;
            w.start = p0;
            w.part = m;
            w.last = m == ns - 1;
            p.work[it0 + m] = w;
        }
    }
    const int64_t used = fits ? total_s : p.N;
    for (int64_t j = used + tid; j < p.max_items; j += 1024) {
        SeqWork w;
        w.seq = 0;
        w.tok0 = 0;
        w.len = -1;
        w.ctx0 = 0;
        w.start = 0;
        w.part = 0;
        w.last = 1;
        p.work[j] = w;
    }
}

// Initial states of the segments of each split sequence, in order:
// S_0 = the sequence's initial state, S_{m+1} = F_m S_m + G_m, in fp32 with
// the products summed in channel order.  One workgroup per (sequence, head,
// 16 state columns); the columns of S evolve independently.
template <int D>
__global__ __launch_bounds__(256) void segment_scan_kernel(PrefillParams p) {
    constexpr int CB = 16, NCB = D / CB, RPT = D / 16, FS = D + 4;
    __shared__ __attribute__((aligned(16))) float F_s[D * FS];
    __shared__ float S_s[D * CB];
    const int H = p.H;
    const int cb = blockIdx.x % NCB;
    const int h = (blockIdx.x / NCB) % H;
    const int seq = blockIdx.x / (NCB * H);
    const int2 si = p.seq_items[seq];
    if (si.y <= 1) return;
    const int tid = threadIdx.x, c = tid % CB, rg = tid / CB;
    const int col = cb * CB + c;
    const int init = p.init_slot ? p.init_slot[seq] : -1;   // in range: only such sequences are cut
    const int64_t ih = (static_cast<int64_t>(init) * H + h) * D * D;
    float acc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; r++) {
        const int64_t e = ih + (rg + 16 * r) * D + col;
        acc[r] = init < 0 ? 0.f
                          : (p.state_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p.state)[e]) << 16)
                                          : static_cast<const float*>(p.state)[e]);
    }
    for (int m = 0;; m++) {
        const int64_t it = static_cast<int64_t>(si.x) + m;
        float* dst = p.seg_S + (it * H + h) * D * D;
#pragma unroll
        for (int r = 0; r < RPT; r++) {
            // a bf16 state pool stores the boundary states rounded: the chain
            // continues from the stored value
            if (p.state_bf16) acc[r] = __uint_as_float(static_cast<uint32_t>(bf16_bits(static_cast<__bf16>(acc[r]))) << 16);
            dst[(rg + 16 * r) * D + col] = acc[r];
            S_s[(rg + 16 * r) * CB + c] = acc[r];
        }
        if (m == si.y - 1) break;
        const float4* Fm = reinterpret_cast<const float4*>(p.seg_F + (it * H + h) * D * D);
        const float* Gm = p.seg_G + (it * H + h) * D * D;
        for (int e = tid; e < D * D / 4; e += 256) {
            const int row = (4 * e) / D, k = (4 * e) % D;
            *reinterpret_cast<float4*>(&F_s[row * FS + k]) = Fm[e];
        }
#pragma unroll
        for (int r = 0; r < RPT; r++) acc[r] = Gm[(rg + 16 * r) * D + col];
        __syncthreads();
        for (int k = 0; k < D; k += 4) {
            const float s0 = S_s[k * CB + c], s1 = S_s[(k + 1) * CB + c];
            const float s2 = S_s[(k + 2) * CB + c], s3 = S_s[(k + 3) * CB + c];
#pragma unroll
            for (int r = 0; r < RPT; r++) {
                const float4 f = *reinterpret_cast<const float4*>(&F_s[(rg + 16 * r) * FS + k]);
                acc[r] = fmaf(f.x, s0, acc[r]);
                acc[r] = fmaf(f.y, s1, acc[r]);
                acc[r] = fmaf(f.z, s2, acc[r]);
                acc[r] = fmaf(f.w, s3, acc[r]);
            }
        }
        __syncthreads();
    }
}

template <int D, typename ACT, bool CD>
hipError_t launch_prefill_t(const PrefillParams& p, hipStream_t s) {
    if (!p.split) {
        const int64_t blocks = static_cast<int64_t>(p.N) * p.H;
        hipLaunchKernelGGL(prefill_meta_kernel, dim3(1), dim3(1024), 0, s, p.cu_seqlens, p.start_pos, p.N, p.T,
                           p.work, p.H, p.ring ? p.ring_ctr : nullptr, p.max_pairs, p.sched_grid, p.status);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (blocks == 0) return hipSuccess;
        if (p.ring) {
            PrefillParams pc = p;
            void* args[] = {&pc};
            const bool all_paired = 2 * blocks <= p.sched_grid && blocks <= p.max_pairs;
            const void* f = all_paired ? reinterpret_cast<const void*>(&prefill_pair_kernel<D, ACT, false, CD>)
                                       : reinterpret_cast<const void*>(&prefill_pair_kernel<D, ACT, true, CD>);
            return hipLaunchCooperativeKernel(f, dim3(static_cast<unsigned>(p.sched_grid)), dim3(4 * D), args, 0, s);
        }
        hipLaunchKernelGGL((prefill_kernel<D, ACT, true, CD>), dim3(static_cast<unsigned>(blocks)), dim3(4 * D), 0, s,
                           p);
        return hipGetLastError();
    }
    const int64_t items = static_cast<int64_t>(p.max_items) * p.H;
    if (p.N == 0 || items == 0) return hipSuccess;
    hipLaunchKernelGGL(prefill_split_meta_kernel, dim3(1), dim3(1024), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_kernel<D, ACT, false, CD>), dim3(static_cast<unsigned>(items)), dim3(4 * D), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(segment_scan_kernel<D>, dim3(static_cast<unsigned>(static_cast<int64_t>(p.N) * p.H * (D / 16))),
                       dim3(256), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((prefill_kernel<D, ACT, true, CD>), dim3(static_cast<unsigned>(items)), dim3(4 * D), 0, s, p);
    return hipGetLastError();
}

}  // namespace

int64_t pair_grid(int64_t chains, int64_t capacity) {
    return min(capacity / 16 * 16, 16 * ((chains + 7) / 8));
}

int64_t prefill_pair_slot_bytes(int dk, int act) {
    if (act == 1) return dk == 32 ? pair_slot_bytes<32, bf16_t>() : dk == 64 ? pair_slot_bytes<64, bf16_t>()
                                                                             : pair_slot_bytes<128, bf16_t>();
    return dk == 32 ? pair_slot_bytes<32, float>() : pair_slot_bytes<64, float>();
}

int64_t prefill_pair_capacity(int dk, int act) {
    const void* f = nullptr;
    if (act == 1) f = dk == 32 ? reinterpret_cast<const void*>(&prefill_pair_kernel<32, bf16_t, true, false>)
                    : dk == 64 ? reinterpret_cast<const void*>(&prefill_pair_kernel<64, bf16_t, true, false>)
                               : reinterpret_cast<const void*>(&prefill_pair_kernel<128, bf16_t, true, false>);
    else f = dk == 32 ? reinterpret_cast<const void*>(&prefill_pair_kernel<32, float, true, false>)
                      : reinterpret_cast<const void*>(&prefill_pair_kernel<64, float, true, false>);
    int dev = 0, cus = 0, per_cu = 0, coop = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, 4 * dk, 0) != hipSuccess) return 0;
    return static_cast<int64_t>(cus) * per_cu;
}

bool prefill_supported(int dk, int dv, int act) {
    if (dk != dv) return false;
    if (act == 1) return dk == 32 || dk == 64 || dk == 128;
    return dk == 32 || dk == 64;   // fp32 activations: raw staging of dk=128 exceeds LDS
}

PrefillWorkspace prefill_workspace(int32_t N, int32_t H, int64_t T, int dk, int dv, int act_bytes,
                                   int32_t ckpt_interval, bool split, bool paired) {
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    PrefillWorkspace w{};
    const int64_t items = split && ckpt_interval > 0 ? 2 * static_cast<int64_t>(N) + T / ckpt_interval : N;
    if (items > INT32_MAX / 4) return w;       // bytes == 0: too many work items
    w.max_items = static_cast<int32_t>(items);
    size_t off = 0;
    w.status = off;                            // int32 status word at byte 0
    off += 256;
    w.items = off;
    off += up(static_cast<size_t>(items) * sizeof(SeqWork));
    if (split) {
        const size_t per = static_cast<size_t>(items) * H;
        w.seq_items = off;
        off += up(static_cast<size_t>(N) * sizeof(int2));
        w.seg_F = off;
        off += up(per * dk * dk * 4);
        w.seg_G = off;
        off += up(per * dk * dv * 4);
        w.seg_S = off;
        off += up(per * dk * dv * 4);
        w.seq_x0 = off;
        off += up(static_cast<size_t>(N) * H * (2 * dk + dv) * 3 * act_bytes);
    }
    const int64_t chains = static_cast<int64_t>(N) * H;
    w.max_pairs = 0;
    if (paired && !split && chains > 0) {
        w.max_pairs = static_cast<int32_t>(min(chains, PAIR_MAX_PAIRS));
        w.ring_ctr = off;
        off += up((static_cast<size_t>(w.max_pairs) * 32 + 32) * 4);
        w.ring = off;
        off += static_cast<size_t>(w.max_pairs) * RING * prefill_pair_slot_bytes(dk, act_bytes == 2 ? 1 : 0);
    }
    w.bytes = off;
    return w;
}

hipError_t launch_prefill(int dk, int dv, int act, const PrefillParams& p, hipStream_t s) {
    if (!prefill_supported(dk, dv, act)) return hipErrorInvalidValue;
    if (act == 1 && p.conv_done) {
        switch (dk) {
            case 32: return launch_prefill_t<32, bf16_t, true>(p, s);
            case 64: return launch_prefill_t<64, bf16_t, true>(p, s);
            default: return launch_prefill_t<128, bf16_t, true>(p, s);
        }
    }
    if (p.conv_done) return hipErrorInvalidValue;          // the conv front end produces bf16 only
    if (act == 1) {
        switch (dk) {
            case 32: return launch_prefill_t<32, bf16_t, false>(p, s);
            case 64: return launch_prefill_t<64, bf16_t, false>(p, s);
            default: return launch_prefill_t<128, bf16_t, false>(p, s);
        }
    }
    return dk == 32 ? launch_prefill_t<32, float, false>(p, s) : launch_prefill_t<64, float, false>(p, s);
}

}  // namespace kda
