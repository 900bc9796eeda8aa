// kda_launch.h -- internal interface between the C ABI (kda_api.cpp) and the
// kernel launchers.  Not installed; the public interface is include/kda.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeParams {
    int32_t B, H, num_slots;
    int32_t T;          // tokens per sequence in this launch (1: one decode step)
    void* token_state;  // [B][T][H][dk][dv] state after every token, or null
    void* token_conv;   // [B][T][H][2dk+dv][3] conv state after every token, or null
    const void* q;
    const void* k;
    const void* v;
    const void* z;
    const float* g;
    const float* beta;
    const float* conv_w;
    const float* norm_w;
    void* state;        // state dtype (fp32 or bf16)
    void* conv;
    const int32_t* slot;
    void* out;
    float l2_eps, rms_eps;
};

struct CopyParams {
    int32_t n, H;
    int64_t state_bytes;   // dk * dv * state element size per head (multiple of 16)
    int64_t conv_bytes;    // (2dk+dv) * 3 * act bytes per head (multiple of 16)
    const void* src_state;
    const void* src_conv;
    int32_t src_slots;
    const int32_t* src_idx;
    void* dst_state;
    void* dst_conv;
    int32_t dst_slots;
    const int32_t* dst_idx;
};

// Work item of the prefill: a whole sequence, or (when sequences are split at
// checkpoint positions) one segment of it.  Built on the device from
// cu_seqlens and start_pos.
struct SeqWork {
    int32_t seq;        // sequence index
    int32_t tok0;       // first packed token of the item
    int32_t len;        // tokens (-1: malformed sequence bounds, skipped)
    int32_t ctx0;       // first packed token of the sequence (conv context before it: initial conv state)
    int64_t start;      // absolute position of the item's first token
    int32_t part;       // index of the item within its sequence (0 when not split)
    int32_t last;       // 1 when the item ends its sequence
};

struct PrefillParams {
    int32_t N, H;
    int64_t T;
    const int32_t* cu_seqlens;
    const int64_t* start_pos;
    const void* q;
    const void* k;
    const void* v;
    const void* z;
    const float* g;
    const float* beta;
    const float* conv_w;
    const float* norm_w;
    void* state;        // state dtype (fp32 or bf16)
    void* conv;
    int32_t num_slots;
    const int32_t* init_slot;
    const int32_t* final_slot;
    int32_t ckpt_interval;
    void* ckpt_state;   // state dtype
    void* ckpt_conv;
    int32_t num_ckpt_slots;
    const int32_t* ckpt_base;
    void* out;
    SeqWork* work;      // work items, in the workspace
    float l2_eps, rms_eps;
    // Sequences split at checkpoint positions (segments run in parallel and
    // are joined by an affine scan of their transitions); all in the workspace.
    int32_t split;      // 0 or 1
    int32_t max_items;  // work items allocated
    int2* seq_items;    // [N] first item and item count per sequence
    float* seg_F;       // [max_items][H][dk][dk] segment transition matrices
    float* seg_G;       // [max_items][H][dk][dv] segment end states from a zero state
    float* seg_S;       // [max_items][H][dk][dv] segment initial states
    void* seq_x0;       // [N][H][2dk+dv][3] initial conv states (activation dtype)
    int32_t state_bf16; // stored state in bf16 (rounded at every store; math in fp32)
    // Scheduled launch (a resident grid; the longest chains get two
    // workgroups each, see prefill_pair_kernel); ring null for the
    // one-workgroup launch.
    char* ring;         // [max_pairs][RING] slots of prefill_pair_slot_bytes each
    int32_t* ring_ctr;  // [max_pairs][32]: chunks handed over at 0, chunks taken at 16; then
                        // [32]: pairs chosen at 0, chain queue at 1
    int32_t max_pairs;  // pairs the ring holds
    int32_t sched_grid; // workgroups of the scheduled launch
    int32_t conv_done;  // q, k, v hold post-conv activations then raw inputs (bf16 only)
    int32_t spin_limit; // polls before a wait between paired workgroups gives up
    int32_t* status;    // workspace word: waits that gave up in this call (zeroed by the metadata kernel)
};

// Input projections: y = x W^T routed to q, k, v, z (activation dtype) and
// g, beta (fp32).
struct ProjectParams {
    int32_t T, N, Dm, H, dk, dv;
    int32_t mode;       // 0: input projections (columns routed to q..beta), 1: plain product into y
    const void* x;      // [T][Dm] bf16
    const void* w;      // [N][Dm] bf16
    void* q;
    void* k;
    void* v;
    void* z;
    void* g;            // fp32
    void* beta;         // fp32
    void* y;            // mode 1: [T][N] bf16
    // conv front end (input projections with the causal conv + SiLU on q, k,
    // v): q, k, v then each point to two tensors back to back, the post-conv
    // activations [T][H][d] and the raw projections [T][H][d]
    int32_t conv;
    int32_t num_seqs;
    const int32_t* cu_seqlens;  // [num_seqs + 1]
    const int32_t* init_slot;   // [num_seqs]: conv-state slot of each sequence's left context, -1 = zero
    const void* conv_pool;      // [num_slots][H][2dk+dv][3] bf16
    int32_t num_slots;
    const float* conv_w;        // [H][2dk+dv][4]
};

// Each launcher returns hipSuccess or the launch error.
hipError_t launch_decode(int dk, int dv, int act, int state, const DecodeParams& p, hipStream_t s);
hipError_t launch_copy(const CopyParams& p, hipStream_t s);
hipError_t launch_project(const ProjectParams& p, hipStream_t s);
hipError_t launch_prefill(int dk, int dv, int act, const PrefillParams& p, hipStream_t s);
bool prefill_supported(int dk, int dv, int act);

// Workspace layout of the prefill (offsets in bytes; total = bytes).
struct PrefillWorkspace {
    int32_t max_items, max_pairs;
    size_t status, items, seq_items, seg_F, seg_G, seg_S, seq_x0, ring_ctr, ring, bytes;
};
// Polls (of 128 cycles each) before a wait between the two workgroups of a
// paired chain gives up: several hundred milliseconds, far above any
// legitimate wait (a chunk takes about 20 us).
constexpr int32_t PAIR_SPIN_LIMIT = 1 << 20;
// A scheduled launch pairs at most this many chains (sequences x heads);
// the ring takes RING slots of prefill_pair_slot_bytes per pair.
constexpr int64_t PAIR_MAX_PAIRS = 256;
PrefillWorkspace prefill_workspace(int32_t N, int32_t H, int64_t T, int dk, int dv, int act_bytes,
                                   int32_t ckpt_interval, bool split, bool paired);
int64_t prefill_pair_slot_bytes(int dk, int act);
// Workgroups of a scheduled launch for this many chains on a device that
// holds `capacity` of them at once (a multiple of 16; 0: none), and that
// capacity for the current device (0 if it cannot tell).
int64_t pair_grid(int64_t chains, int64_t capacity);
int64_t prefill_pair_capacity(int dk, int act);

// Record an error message for kda_last_error() on this thread (printf-style)
// and return st; for entry points defined outside kda_api.cpp.
int set_error(int st, const char* fmt, ...);

}  // namespace kda
