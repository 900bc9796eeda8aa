// decode.hip -- fused single-launch KDA decode step for gfx950.
//
// One workgroup per (sequence, head).  The dk x dv state of the pair is
// streamed from HBM once into registers (128-bit loads for an fp32 state,
// 64-bit for a bf16 one), updated there in fp32 and streamed back once; everything else (conv-state shift, causal conv + SiLU,
// L2 norms, decay, delta update, readout, gated RMSNorm) happens while the
// state loads are in flight or on registers/LDS, in the same launch.
// [vLLM blog "A Preview of Production-Scale Kimi K3 Support on vLLM", section
//  "KDA prefill and decode": decode runs the short convolution, state update,
//  output gate and normalisation together rather than as separate launches;
//  agentlenshq "vLLM Kimi K3 Support", section "Fused Kernels and Metadata
//  Optimization": a single launch avoids intermediate tensors and repeated
//  state traffic.]
//
// Thread layout: the dv columns are split into NCG groups of 4 (one float4
// per row), the dk rows into RG blocks of RPT consecutive rows; thread
// (rg, cg) owns rows rg*RPT .. rg*RPT+RPT-1 and columns 4cg..4cg+3, i.e. RPT
// float4 registers.  Each load instruction of a wave reads whole rows
// (NCG lanes x 16 bytes per row).  The two dk-reductions (S'^T k and S'^T q) go
// through the thread's rows, then lane moves across row groups of a wave
// (DPP and row swaps, no LDS), then LDS across waves.
//
// The readout uses o = S^T q = S'^T q + u (q . k) (S' the decayed state,
// u the delta-rule update), so the state is read once and written once.

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// ST: stored state type (float, or bf16_t: loaded to fp32, rounded to nearest
// bf16 on the store; the math is fp32 either way).
template <int DK, int DV, typename ACT, typename ST, int NT>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeParams p) {
    constexpr int NCG = DV / 4;
    constexpr int RG = NT / NCG;
    constexpr int RPT = DK / RG;
    constexpr int NW = NT / 64;
    constexpr int C = 2 * DK + DV;
    constexpr int CPT = (C + NT - 1) / NT;  // conv channels per thread
    static_assert(NCG <= 64 && 64 % NCG == 0, "column groups must tile a wave");
    static_assert(RG * NCG == NT && RPT * RG == DK, "rows must tile the workgroup");
    static_assert(DK <= NT, "one thread per key channel for the gate");
    using A = Act<ACT>;

    __shared__ float a_s[C];            // SiLU(conv(x)) for q | k | v
    __shared__ float eg_s[DK];          // exp(g)
    __shared__ float red_s[NW][2][DV];  // per-wave partial S'^T k and S'^T q
    __shared__ float nrm_s[NW][3];      // per-wave partial |a_q|^2, |a_k|^2, a_q.a_k

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int cg = tid % NCG, rg = tid / NCG;
    const int H = p.H;
    const int b = blockIdx.x / H, h = blockIdx.x % H;
    const int64_t bh = static_cast<int64_t>(b) * H + h;

    ACT* out = static_cast<ACT*>(p.out) + bh * DV;
    const int slot = p.slot[b];
    if (slot < 0 || slot >= p.num_slots) {
        for (int j = tid; j < DV; j += NT) A::st(out + j, nan_f32());
        return;
    }
    const int64_t sh = static_cast<int64_t>(slot) * H + h;

    // 1. small operands first, as raw bits and with unconditional (clamped)
    // addresses.  Vector-memory waits complete in issue order, so everything
    // the prologue and epilogue need is requested before the state and
    // converted only after the state loads are in flight.
    const ACT* xq = static_cast<const ACT*>(p.q) + bh * DK;
    const ACT* xk = static_cast<const ACT*>(p.k) + bh * DK;
    const ACT* xv = static_cast<const ACT*>(p.v) + bh * DV;
    ACT* X = static_cast<ACT*>(p.conv) + sh * C * 3;
    const float* w = p.conv_w + static_cast<int64_t>(h) * C * 4;
    typename A::raw xin[CPT], x0[CPT], x1[CPT], x2[CPT];
    float4 wc[CPT];
#pragma unroll
    for (int j = 0; j < CPT; j++) {
        const int c = min(tid + j * NT, C - 1);
        const ACT* src = c < DK ? xq + c : (c < 2 * DK ? xk + (c - DK) : xv + (c - 2 * DK));
        xin[j] = A::ld_raw(src);
        x0[j] = A::ld_raw(X + c * 3);
        x1[j] = A::ld_raw(X + c * 3 + 1);
        x2[j] = A::ld_raw(X + c * 3 + 2);
        wc[j] = *reinterpret_cast<const float4*>(w + c * 4);
    }
    const float gv = p.g[bh * DK + min(tid, DK - 1)];
    const float bt = p.beta[bh];
    const float4 nw = *reinterpret_cast<const float4*>(p.norm_w + 4 * cg);
    const typename A::raw4 zraw = A::ld4_raw(static_cast<const ACT*>(p.z) + bh * DV + 4 * cg);

    // 2. the state: RPT consecutive rows x 4 columns per thread, through a
    // buffer resource covering this (slot, head) only
    __builtin_amdgcn_sched_barrier(0);
    constexpr uint32_t SB = sizeof(ST);
    const auto rs = make_rsrc(static_cast<ST*>(p.state) + sh * DK * DV, DK * DV * SB);
    const uint32_t voff = static_cast<uint32_t>((rg * RPT * DV + 4 * cg) * SB);
    float4 s[RPT];
#pragma unroll
    for (int r = 0; r < RPT; r++) {
        if constexpr (SB == 4) s[r] = buf_ld4(rs, voff + (r % 8) * DV * 4, (r / 8) * 8 * DV * 4);
        else s[r] = bf16x4_to_f32(buf_ld8(rs, voff + r * DV * 2));
    }
    __builtin_amdgcn_sched_barrier(0);

    // 3. conv-state shift + causal depthwise conv (width 4) + SiLU
#pragma unroll
    for (int j = 0; j < CPT; j++) {
        const int c = tid + j * NT;
        if (c < C) {
            const float f0 = A::cvt(x0[j]), f1 = A::cvt(x1[j]), f2 = A::cvt(x2[j]), fx = A::cvt(xin[j]);
            float y = wc[j].x * f0;
            y = fmaf(wc[j].y, f1, y);
            y = fmaf(wc[j].z, f2, y);
            y = fmaf(wc[j].w, fx, y);
            a_s[c] = silu(y);
            ACT* xs = X + c * 3;
            reinterpret_cast<typename A::raw*>(xs)[0] = x1[j];
            reinterpret_cast<typename A::raw*>(xs)[1] = x2[j];
            reinterpret_cast<typename A::raw*>(xs)[2] = xin[j];
        }
    }
    if (tid < DK) eg_s[tid] = __expf(gv);
    __syncthreads();

    // 4. L2 norms of q and k, and q.k
    float pq = 0.f, pk = 0.f, pqk = 0.f;
    for (int i = tid; i < DK; i += NT) {
        const float aq = a_s[i], ak = a_s[DK + i];
        pq = fmaf(aq, aq, pq);
        pk = fmaf(ak, ak, pk);
        pqk = fmaf(aq, ak, pqk);
    }
    pq = lane_sum_below<64>(pq);
    pk = lane_sum_below<64>(pk);
    pqk = lane_sum_below<64>(pqk);
    if (lane == 0) {
        nrm_s[wave][0] = pq;
        nrm_s[wave][1] = pk;
        nrm_s[wave][2] = pqk;
    }
    __syncthreads();
    float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; w2++) {
        sq += nrm_s[w2][0];
        sk += nrm_s[w2][1];
        sqk += nrm_s[w2][2];
    }
    const float rq = rsqrtf(sq + p.l2_eps);
    const float rk = rsqrtf(sk + p.l2_eps);
    const float qk = sqk * rq * rk;

    // 5. decay, then the two reductions over the decayed rows
    float4 pred = make_float4(0.f, 0.f, 0.f, 0.f), rr = pred;
#pragma unroll
    for (int r = 0; r < RPT; r++) {
        const int i = rg * RPT + r;
        const float e = eg_s[i];
        const float kh = a_s[DK + i] * rk;
        const float qh = a_s[i] * rq;
        s[r].x *= e; s[r].y *= e; s[r].z *= e; s[r].w *= e;
        pred.x = fmaf(s[r].x, kh, pred.x); pred.y = fmaf(s[r].y, kh, pred.y);
        pred.z = fmaf(s[r].z, kh, pred.z); pred.w = fmaf(s[r].w, kh, pred.w);
        rr.x = fmaf(s[r].x, qh, rr.x); rr.y = fmaf(s[r].y, qh, rr.y);
        rr.z = fmaf(s[r].z, qh, rr.z); rr.w = fmaf(s[r].w, qh, rr.w);
    }
    pred.x = lane_sum_from<NCG>(pred.x); pred.y = lane_sum_from<NCG>(pred.y);
    pred.z = lane_sum_from<NCG>(pred.z); pred.w = lane_sum_from<NCG>(pred.w);
    rr.x = lane_sum_from<NCG>(rr.x); rr.y = lane_sum_from<NCG>(rr.y);
    rr.z = lane_sum_from<NCG>(rr.z); rr.w = lane_sum_from<NCG>(rr.w);
    if (lane < NCG) {
        *reinterpret_cast<float4*>(&red_s[wave][0][4 * cg]) = pred;
        *reinterpret_cast<float4*>(&red_s[wave][1][4 * cg]) = rr;
    }
    __syncthreads();
    pred = *reinterpret_cast<const float4*>(&red_s[0][0][4 * cg]);
    rr = *reinterpret_cast<const float4*>(&red_s[0][1][4 * cg]);
#pragma unroll
    for (int w2 = 1; w2 < NW; w2++) {
        const float4 a = *reinterpret_cast<const float4*>(&red_s[w2][0][4 * cg]);
        const float4 c = *reinterpret_cast<const float4*>(&red_s[w2][1][4 * cg]);
        pred.x += a.x; pred.y += a.y; pred.z += a.z; pred.w += a.w;
        rr.x += c.x; rr.y += c.y; rr.z += c.z; rr.w += c.w;
    }

    // 6. delta update u = beta (v - S'^T k), readout o = S'^T q + u (q.k)
    const float4 vh = *reinterpret_cast<const float4*>(&a_s[2 * DK + 4 * cg]);
    float4 u, o;
    u.x = bt * (vh.x - pred.x); u.y = bt * (vh.y - pred.y);
    u.z = bt * (vh.z - pred.z); u.w = bt * (vh.w - pred.w);
    o.x = fmaf(u.x, qk, rr.x); o.y = fmaf(u.y, qk, rr.y);
    o.z = fmaf(u.z, qk, rr.z); o.w = fmaf(u.w, qk, rr.w);

    // 7. S = S' + k u^T, written back once
#pragma unroll
    for (int r = 0; r < RPT; r++) {
        const float kh = a_s[DK + rg * RPT + r] * rk;
        s[r].x = fmaf(kh, u.x, s[r].x); s[r].y = fmaf(kh, u.y, s[r].y);
        s[r].z = fmaf(kh, u.z, s[r].z); s[r].w = fmaf(kh, u.w, s[r].w);
        if constexpr (SB == 4) buf_st4(rs, voff + r * DV * 4, s[r]);
        else buf_st8(rs, voff + r * DV * 2, f32_to_bf16x4(s[r]));
    }

    // 8. gated RMSNorm over dv (every row group holds all of o)
    float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
    ss = lane_sum_below<NCG>(ss);
    if (rg == 0) {
        const float rinv = rsqrtf(ss * (1.0f / DV) + p.rms_eps);
        const float4 zz = A::cvt4(zraw);
        float4 y;
        y.x = o.x * rinv * nw.x * sigmoid(zz.x);
        y.y = o.y * rinv * nw.y * sigmoid(zz.y);
        y.z = o.z * rinv * nw.z * sigmoid(zz.z);
        y.w = o.w * rinv * nw.w * sigmoid(zz.w);
        A::st4(out + 4 * cg, y);
    }
}

// Non-temporal 16- and 8-byte stores (cache-policy bit NT): for data written
// once and not read again by this launch or the next (the per-token rollback
// states of a multi-token step).  Without the hint that stream takes the place
// of the live state in the last-level cache and the next step reads the state
// from HBM again.  Bit 1 of the intrinsics' cache-policy operand is NT on gfx950.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void buf_st4_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, float4 x) {
    i32x4 v;
    v.x = __float_as_int(x.x);
    v.y = __float_as_int(x.y);
    v.z = __float_as_int(x.z);
    v.w = __float_as_int(x.w);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, static_cast<int>(voff), 0, kCachePolicyNT);
}
__device__ __forceinline__ void buf_st8_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint2 x) {
    i32x2 v;
    v.x = static_cast<int>(x.x);
    v.y = static_cast<int>(x.y);
    __builtin_amdgcn_raw_buffer_store_b64(v, r, static_cast<int>(voff), 0, kCachePolicyNT);
}

// T decode tokens per sequence in one launch (speculative verification: the
// target model checks K drafted tokens plus one in a single pass).  The state
// stays in registers across the tokens; token t runs exactly the arithmetic
// of one decode_kernel step (with a bf16 state, the state is rounded after
// every token, as a store and reload between steps would), so the results
// equal T single-token launches bit for bit.  Optionally the state and conv
// state after every token are written to token_state / token_conv (slot
// b*T + t), from which a rejected draft is rolled back by a slot copy.
// [agentlenshq "vLLM Kimi K3 Support", section "Speculative Decoding with
//  DSpark": vLLM serves the model with a drafting speculator; vLLM recipe
//  "moonshotai/Kimi-K3", section "AMD MI355X: disaggregated prefill and
//  decode": the decode worker drafts four tokens per step.]
template <int DK, int DV, typename ACT, typename ST, int NT>
__global__ __launch_bounds__(NT) void decode_multi_kernel(DecodeParams p) {
    constexpr int NCG = DV / 4;
    constexpr int RG = NT / NCG;
    constexpr int RPT = DK / RG;
    constexpr int NW = NT / 64;
    constexpr int C = 2 * DK + DV;
    constexpr int CPT = (C + NT - 1) / NT;
    using A = Act<ACT>;
    constexpr uint32_t SB = sizeof(ST);

    __shared__ float a_s[C];
    __shared__ float eg_s[DK];
    __shared__ float red_s[NW][2][DV];
    __shared__ float nrm_s[NW][3];
    // the small per-token operands of up to TG tokens, staged together so that
    // one memory round trip serves TG tokens (the compute of one token is
    // shorter than a round trip to HBM): per token q | k | v | z (ACT) then
    // g (DK fp32) and beta (fp32, padded to 16 bytes)
    constexpr int TG = 8;
    constexpr int QC = DK * A::kBytes / 16, VC = DV * A::kBytes / 16, GC = DK * 4 / 16;
    constexpr int OPC = 2 * QC + 2 * VC + GC;          // 16-byte chunks of one token
    constexpr int OPB = OPC * 16;                       // bytes of one token's operands
    static_assert(DK * A::kBytes % 16 == 0 && DV * A::kBytes % 16 == 0, "rows must be 16-byte multiples");
    __shared__ __attribute__((aligned(16))) char op_s[TG * OPB];
    __shared__ float bt_s[TG];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int cg = tid % NCG, rg = tid / NCG;
    const int H = p.H, B = p.B, T = p.T;
    const int b = blockIdx.x / H, h = blockIdx.x % H;
    const int64_t bh = static_cast<int64_t>(b) * H + h;
    const int64_t step = static_cast<int64_t>(B) * H;     // one token of every (sequence, head)

    ACT* out = static_cast<ACT*>(p.out) + bh * DV;
    const int slot = p.slot[b];
    if (slot < 0 || slot >= p.num_slots) {
        for (int t = 0; t < T; t++)
            for (int j = tid; j < DV; j += NT) A::st(out + t * step * DV + j, nan_f32());
        return;
    }
    const int64_t sh = static_cast<int64_t>(slot) * H + h;

    // operands of tokens t0 .. t0 + n - 1 into op_s, straight from global
    // memory into LDS (16 bytes per lane; a wave instruction fills 1 KiB of
    // consecutive chunks), no registers holding them; visible after the
    // caller's wait and barrier
    auto stage = [&](int t0, int n, int ln) {
        constexpr int PER = (TG * OPC + NT - 1) / NT;
#pragma unroll
        for (int i = 0; i < PER; i++) {
            const int e0 = (i * NW + wave) * 64;        // first chunk of this wave instruction
            const int e = e0 + ln;
            if (e0 < n * OPC && e < n * OPC) {
                const int tt = e / OPC, c = e % OPC;
                const int64_t row = (t0 + tt) * step + bh;
                const uint4* src =
                    c < QC ? reinterpret_cast<const uint4*>(static_cast<const ACT*>(p.q) + row * DK) + c
                    : c < 2 * QC ? reinterpret_cast<const uint4*>(static_cast<const ACT*>(p.k) + row * DK) + (c - QC)
                    : c < 2 * QC + VC ? reinterpret_cast<const uint4*>(static_cast<const ACT*>(p.v) + row * DV) + (c - 2 * QC)
                    : c < 2 * QC + 2 * VC ? reinterpret_cast<const uint4*>(static_cast<const ACT*>(p.z) + row * DV) + (c - 2 * QC - VC)
                    : reinterpret_cast<const uint4*>(p.g + row * DK) + (c - 2 * QC - 2 * VC);
                __builtin_amdgcn_global_load_lds(src, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                                          reinterpret_cast<uintptr_t>(op_s + e0 * 16)),
                                                 16, 0, 0);
            }
        }
        if (tid < n) bt_s[tid] = p.beta[(t0 + tid) * step + bh];
    };
    stage(0, min(T, TG), lane);

    // conv window (raw, oldest first) and weights
    ACT* X = static_cast<ACT*>(p.conv) + sh * C * 3;
    const float* w = p.conv_w + static_cast<int64_t>(h) * C * 4;
    typename A::raw x0[CPT], x1[CPT], x2[CPT];
    float4 wc[CPT];
#pragma unroll
    for (int j = 0; j < CPT; j++) {
        const int c = min(tid + j * NT, C - 1);
        x0[j] = A::ld_raw(X + c * 3);
        x1[j] = A::ld_raw(X + c * 3 + 1);
        x2[j] = A::ld_raw(X + c * 3 + 2);
        wc[j] = *reinterpret_cast<const float4*>(w + c * 4);
    }
    const float4 nw = *reinterpret_cast<const float4*>(p.norm_w + 4 * cg);

    __builtin_amdgcn_sched_barrier(0);
    const auto rs = make_rsrc(static_cast<ST*>(p.state) + sh * DK * DV, DK * DV * SB);
    const uint32_t voff = static_cast<uint32_t>((rg * RPT * DV + 4 * cg) * SB);
    // the state: fp32 in s; a bf16 state stays packed in sp between tokens
    // (after every token it is exactly its bf16 rounding), which halves its
    // registers.  Within a token its rows are widened and decayed in the
    // reductions and kept in xd for the update (KEEP), or, where those 64
    // values would cost a wave per SIMD (fp32 activations at d = 128), widened
    // and decayed again in the update; the values are those of the fp32 form
    constexpr int RS = SB == 4 ? RPT : 1, RP = SB == 2 ? RPT : 1;
    constexpr bool KEEP = SB == 2 && !(sizeof(ACT) == 4 && DK == 128);
    float4 s[RS];
    uint2 sp[RP];
#pragma unroll
    for (int r = 0; r < RPT; r++) {
        if constexpr (SB == 4) s[r] = buf_ld4(rs, voff + (r % 8) * DV * 4, (r / 8) * 8 * DV * 4);
        else sp[r] = buf_ld8(rs, voff + r * DV * 2);
    }
    __builtin_amdgcn_sched_barrier(0);
    auto decayed = [&](int r, float e) -> float4 {
        float4 x;
        if constexpr (SB == 4) x = s[r];
        else x = bf16x4_to_f32(sp[r]);
        x.x *= e; x.y *= e; x.z *= e; x.w *= e;
        return x;
    };

    for (int t = 0; t < T; t++) {
        if (t % TG == 0) {
            // every wave is past the previous group's last token (its closing
            // barrier), so its slots may be overwritten
            if (t > 0) {
                // the lane index made opaque here, so that the copies' address
                // arithmetic is formed in place rather than hoisted out of the
                // token loop into live registers (no instruction emitted)
                int ln = lane;
                asm volatile("" : "+v"(ln));
                stage(t, min(T - t, TG), ln);
            }
            __builtin_amdgcn_s_waitcnt(0);              // this wave's copies have landed
            __syncthreads();
        }
        const char* op = op_s + (t % TG) * OPB;
        const ACT* op_a = reinterpret_cast<const ACT*>(op);      // q | k | v | z: conv channel c at c
        typename A::raw xin[CPT];
#pragma unroll
        for (int j = 0; j < CPT; j++) xin[j] = A::ld_raw(op_a + min(tid + j * NT, C - 1));
        const float gv = reinterpret_cast<const float*>(op + (2 * QC + 2 * VC) * 16)[min(tid, DK - 1)];
        const float bt = bt_s[t % TG];
        const typename A::raw4 zraw = A::ld4_raw(op_a + 2 * DK + DV + 4 * cg);

        // conv + SiLU; the window shifts in registers
#pragma unroll
        for (int j = 0; j < CPT; j++) {
            const int c = tid + j * NT;
            if (c < C) {
                const float f0 = A::cvt(x0[j]), f1 = A::cvt(x1[j]), f2 = A::cvt(x2[j]), fx = A::cvt(xin[j]);
                float y = wc[j].x * f0;
                y = fmaf(wc[j].y, f1, y);
                y = fmaf(wc[j].z, f2, y);
                y = fmaf(wc[j].w, fx, y);
                a_s[c] = silu(y);
            }
            x0[j] = x1[j];
            x1[j] = x2[j];
            x2[j] = xin[j];
        }
        if (p.token_conv) {
            ACT* tc = static_cast<ACT*>(p.token_conv) + ((static_cast<int64_t>(b) * T + t) * H + h) * C * 3;
#pragma unroll
            for (int j = 0; j < CPT; j++) {
                const int c = tid + j * NT;
                if (c < C) {
                    reinterpret_cast<typename A::raw*>(tc + c * 3)[0] = x0[j];
                    reinterpret_cast<typename A::raw*>(tc + c * 3)[1] = x1[j];
                    reinterpret_cast<typename A::raw*>(tc + c * 3)[2] = x2[j];
                }
            }
        }
        if (tid < DK) eg_s[tid] = __expf(gv);
        __syncthreads();

        // L2 norms of q and k, and q.k
        float pq = 0.f, pk = 0.f, pqk = 0.f;
        for (int i = tid; i < DK; i += NT) {
            const float aq = a_s[i], ak = a_s[DK + i];
            pq = fmaf(aq, aq, pq);
            pk = fmaf(ak, ak, pk);
            pqk = fmaf(aq, ak, pqk);
        }
        pq = lane_sum_below<64>(pq);
        pk = lane_sum_below<64>(pk);
        pqk = lane_sum_below<64>(pqk);
        if (lane == 0) {
            nrm_s[wave][0] = pq;
            nrm_s[wave][1] = pk;
            nrm_s[wave][2] = pqk;
        }
        __syncthreads();
        float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; w2++) {
            sq += nrm_s[w2][0];
            sk += nrm_s[w2][1];
            sqk += nrm_s[w2][2];
        }
        const float rq = rsqrtf(sq + p.l2_eps);
        const float rk = rsqrtf(sk + p.l2_eps);
        const float qk = sqk * rq * rk;

        // decay, then the two reductions over the decayed rows
        float4 pred = make_float4(0.f, 0.f, 0.f, 0.f), rr = pred;
        float4 xd[KEEP ? RPT : 1];
#pragma unroll
        for (int r = 0; r < RPT; r++) {
            const int i = rg * RPT + r;
            const float e = eg_s[i];
            const float kh = a_s[DK + i] * rk;
            const float qh = a_s[i] * rq;
            const float4 x = decayed(r, e);
            if constexpr (SB == 4) s[r] = x;
            if constexpr (KEEP) xd[r] = x;
            pred.x = fmaf(x.x, kh, pred.x); pred.y = fmaf(x.y, kh, pred.y);
            pred.z = fmaf(x.z, kh, pred.z); pred.w = fmaf(x.w, kh, pred.w);
            rr.x = fmaf(x.x, qh, rr.x); rr.y = fmaf(x.y, qh, rr.y);
            rr.z = fmaf(x.z, qh, rr.z); rr.w = fmaf(x.w, qh, rr.w);
        }
        if constexpr (SB == 2 && !KEEP) {
            // widen again in the update below rather than keep the decayed
            // fp32 rows alive across the reductions (no instruction emitted)
#pragma unroll
            for (int r = 0; r < RPT; r++) asm volatile("" : "+v"(sp[r].x), "+v"(sp[r].y));
        }
        pred.x = lane_sum_from<NCG>(pred.x); pred.y = lane_sum_from<NCG>(pred.y);
        pred.z = lane_sum_from<NCG>(pred.z); pred.w = lane_sum_from<NCG>(pred.w);
        rr.x = lane_sum_from<NCG>(rr.x); rr.y = lane_sum_from<NCG>(rr.y);
        rr.z = lane_sum_from<NCG>(rr.z); rr.w = lane_sum_from<NCG>(rr.w);
        if (lane < NCG) {
            *reinterpret_cast<float4*>(&red_s[wave][0][4 * cg]) = pred;
            *reinterpret_cast<float4*>(&red_s[wave][1][4 * cg]) = rr;
        }
        __syncthreads();
        pred = *reinterpret_cast<const float4*>(&red_s[0][0][4 * cg]);
        rr = *reinterpret_cast<const float4*>(&red_s[0][1][4 * cg]);
#pragma unroll
        for (int w2 = 1; w2 < NW; w2++) {
            const float4 a = *reinterpret_cast<const float4*>(&red_s[w2][0][4 * cg]);
            const float4 c = *reinterpret_cast<const float4*>(&red_s[w2][1][4 * cg]);
            pred.x += a.x; pred.y += a.y; pred.z += a.z; pred.w += a.w;
            rr.x += c.x; rr.y += c.y; rr.z += c.z; rr.w += c.w;
        }

        // delta update and readout
        const float4 vh = *reinterpret_cast<const float4*>(&a_s[2 * DK + 4 * cg]);
        float4 u, o;
        u.x = bt * (vh.x - pred.x); u.y = bt * (vh.y - pred.y);
        u.z = bt * (vh.z - pred.z); u.w = bt * (vh.w - pred.w);
        o.x = fmaf(u.x, qk, rr.x); o.y = fmaf(u.y, qk, rr.y);
        o.z = fmaf(u.z, qk, rr.z); o.w = fmaf(u.w, qk, rr.w);

        // S = S' + k u^T (rounded to the stored dtype: the next token starts
        // from what a store would hold), optionally kept for rollback
        const auto rt = make_rsrc(p.token_state ? static_cast<ST*>(p.token_state) +
                                                      ((static_cast<int64_t>(b) * T + t) * H + h) * DK * DV
                                                : static_cast<ST*>(p.state),
                                  p.token_state ? DK * DV * SB : 0u);
        // the row offsets are formed here from an offset the compiler cannot
        // hoist: hoisted out of the token loop they became RPT live VGPRs,
        // here they fold into the stores' immediate offset field
        uint32_t vo = voff;
        asm volatile("" : "+v"(vo));
#pragma unroll
        for (int r = 0; r < RPT; r++) {
            const float kh = a_s[DK + rg * RPT + r] * rk;
            float4 x = SB == 4 ? s[RS > 1 ? r : 0] : (KEEP ? xd[KEEP ? r : 0] : decayed(r, eg_s[rg * RPT + r]));
            x.x = fmaf(kh, u.x, x.x); x.y = fmaf(kh, u.y, x.y);
            x.z = fmaf(kh, u.z, x.z); x.w = fmaf(kh, u.w, x.w);
            if constexpr (SB == 2) {
                sp[r] = f32_to_bf16x4(x);
                if (p.token_state) buf_st8_nt(rt, vo + r * DV * 2, sp[r]);
            } else {
                s[r] = x;
                if (p.token_state) buf_st4_nt(rt, vo + r * DV * 4, s[r]);
            }
        }

        // gated RMSNorm over dv
        float ss = o.x * o.x + o.y * o.y + o.z * o.z + o.w * o.w;
        ss = lane_sum_below<NCG>(ss);
        if (rg == 0) {
            const float rinv = rsqrtf(ss * (1.0f / DV) + p.rms_eps);
            const float4 zz = A::cvt4(zraw);
            float4 y;
            y.x = o.x * rinv * nw.x * sigmoid(zz.x);
            y.y = o.y * rinv * nw.y * sigmoid(zz.y);
            y.z = o.z * rinv * nw.z * sigmoid(zz.z);
            y.w = o.w * rinv * nw.w * sigmoid(zz.w);
            A::st4(out + t * step * DV + 4 * cg, y);
        }
        __syncthreads();        // a_s, eg_s and the reduction buffers are reused
    }

    // final state and conv window to the pool
#pragma unroll
    for (int r = 0; r < RPT; r++) {
        if constexpr (SB == 4) buf_st4(rs, voff + r * DV * 4, s[r]);
        else buf_st8(rs, voff + r * DV * 2, sp[r]);
    }
#pragma unroll
    for (int j = 0; j < CPT; j++) {
        const int c = tid + j * NT;
        if (c < C) {
            reinterpret_cast<typename A::raw*>(X + c * 3)[0] = x0[j];
            reinterpret_cast<typename A::raw*>(X + c * 3)[1] = x1[j];
            reinterpret_cast<typename A::raw*>(X + c * 3)[2] = x2[j];
        }
    }
}

template <int DK, int DV, typename ACT, typename ST, int NT>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(p.B) * p.H;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_kernel<DK, DV, ACT, ST, NT>), dim3(static_cast<unsigned>(blocks)),
                       dim3(NT), 0, s, p);
    return hipGetLastError();
}

template <int DK, int DV, typename ACT, typename ST, int NT>
static hipError_t launch_decode_multi_t(const DecodeParams& p, hipStream_t s) {
    const int64_t blocks = static_cast<int64_t>(p.B) * p.H;
    if (blocks == 0 || p.T == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_multi_kernel<DK, DV, ACT, ST, NT>), dim3(static_cast<unsigned>(blocks)),
                       dim3(NT), 0, s, p);
    return hipGetLastError();
}

template <typename ACT, typename ST>
static hipError_t launch_decode_d(int d, const DecodeParams& p, hipStream_t s) {
    const bool multi = p.T != 1 || p.token_state || p.token_conv;
    switch (d) {
        case 32:  return multi ? launch_decode_multi_t<32, 32, ACT, ST, 64>(p, s) : launch_decode_t<32, 32, ACT, ST, 64>(p, s);
        case 64:  return multi ? launch_decode_multi_t<64, 64, ACT, ST, 128>(p, s) : launch_decode_t<64, 64, ACT, ST, 128>(p, s);
        case 128: return multi ? launch_decode_multi_t<128, 128, ACT, ST, 256>(p, s) : launch_decode_t<128, 128, ACT, ST, 256>(p, s);
        default:  return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(int dk, int dv, int act, int state, const DecodeParams& p, hipStream_t s) {
    if (dk != dv) return hipErrorInvalidValue;
    if (act == 1) return state == 1 ? launch_decode_d<bf16_t, bf16_t>(dk, p, s) : launch_decode_d<bf16_t, float>(dk, p, s);
    return state == 1 ? launch_decode_d<float, bf16_t>(dk, p, s) : launch_decode_d<float, float>(dk, p, s);
}

}  // namespace kda
