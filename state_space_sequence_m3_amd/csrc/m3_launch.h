// m3_launch.h -- argument blocks and launchers shared between the C-ABI layer and the kernels.
// Shapes and pointers are validated by the C-ABI layer (api.hip) before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m3 {

struct DecodeArgs {
    float* h;
    const void* Bbar_prev;
    const void* x_prev;
    const void* x;
    const void* Bbar;
    const void* Cbar;
    const void* dt;
    const float* A;
    const void* lam;
    const float* w_out;
    void* y;
    int64_t b;
    int H, N, P, R;
    // fused step only (launch_layer_decode): Bbar and Cbar above then point at the raw B and C of
    // the token, which the kernel normalises, biases and rotates by the carried angle first
    const void* theta = nullptr;
    const float* normw_B = nullptr;
    const float* normw_C = nullptr;
    const float* bias_B = nullptr;
    const float* bias_C = nullptr;
    float* phi = nullptr;        // [b, H, N/2] in/out
    void* Bbar_out = nullptr;    // [b, H, R, N] the token's rotated B (next step's Bbar_prev)
    int bcnorm = 0;
    float eps = 0.f;
    // raw B and C hold G head slots: head h reads slot h / (H / G) (0: one slot per head)
    int G = 0;
};

struct BcnormRopeArgs {
    const void* B;
    const void* C;
    const void* dt;
    const void* theta;
    const float* normw_B;
    const float* normw_C;
    const float* bias_B;
    const float* bias_C;
    const float* phi_in;
    float* seg_phi;       // [b, H, nseg, parts, N/2] quarter start angles (nseg > 1), else nullptr
    void* Bbar;
    void* Cbar;
    float* phi_out;
    int64_t b, L;
    int H, N, R;
    int64_t seglen;       // time steps per segment
    int nseg;             // segments per (b, h)
    int bcnorm;
    float eps;
    // raw B and C hold G head slots: head h reads slot h / (H / G) (0: one slot per head)
    int G = 0;
};

struct PrefillArgs {
    const void* x;
    const void* Bbar;
    const void* Cbar;
    const void* dt;
    const float* A;
    const void* lam;
    const float* w_out;
    const float* h_in;
    const void* Bbar_prev;
    const void* x_prev;
    void* y;
    float* h_out;
    void* Bbar_last;
    void* x_last;
    int64_t b, L;
    int H, N, P, R;
    int Q;                // time steps per chunk; Q * R rows per chunk tile (16..64)
    // fused layer only (launch_layer): Bbar and Cbar above then point at the raw B and C, which
    // the kernel normalises, biases and rotates while staging each chunk
    const void* theta = nullptr;
    const float* normw_B = nullptr;
    const float* normw_C = nullptr;
    const float* bias_B = nullptr;
    const float* bias_C = nullptr;
    const float* phi_in = nullptr;
    float* phi_out = nullptr;
    int bcnorm = 0;
    float eps = 0.f;
    // packed variable-length batch: sequence s holds tokens [cu_seqlens[s], cu_seqlens[s+1]) of
    // T packed tokens (b = number of sequences); nullptr = dense [b, L, ...]
    const int32_t* cu_seqlens = nullptr;
    int64_t T = 0;
    // Sequence split (few (b, h) pairs, long sequences): each sequence is cut into nseg segments
    // of seglen steps.  pass 0 = no split.  pass 1 runs every segment at once, segment 0 from the
    // call's carry (state, last step, angle) and the others from zero, writing y, each segment's
    // end state, last Bbar row, log2 decay, end angle (fused) and ws_fix (the steps from the
    // segment's start after which the carried-in state's share of y, which decays as 2^l2, stays
    // below 2^-48 of its size), and the call's x_last from the last segment; segment_combine
    // chains the end angles into true start angles, turns the later segments' end states and
    // Bbar rows to them, chains the end states (leaving in each segment's slot the state that
    // enters the next one), and writes h_out, Bbar_last and phi_out; pass 2 reruns the first
    // ws_fix steps of segments 1 .. nseg-1 from their entering state and true start angle,
    // writing y only.
    int pass = 0;
    int nseg = 1;
    int64_t seglen = 0;
    float* ws_state = nullptr;       // [b, H, nseg, N, P] end state of each segment (pass 1)
    void* ws_bbar = nullptr;         // [b, H, nseg, R, N] io, Bbar of each segment's last step (pass 1)
    float* ws_l2 = nullptr;          // [b, H, nseg] log2 decay of each segment (log2 e A sum of dt)
    int* ws_fix = nullptr;           // [b, H, nseg] pass 1 -> pass 2: steps of each segment to rerun
    float* ws_phiend = nullptr;      // fused: [b, H, nseg, N/2] end angle of each segment in pass 1
                                     // (radians; segment 0 true, the others from zero)
    float* seg_phi = nullptr;        // fused: [b, H, nseg, N/2] true start angle of each segment
    // fused layer only: raw B and C hold G head slots, head h reads slot h / (H / G) (0: one slot
    // per head); the heads of a group are then laid out on one XCD (see xcd_block)
    int G = 0;
};

// Gradients of the fused layer core (m3_layer_chunk_states / m3_layer_backward).  B and C are raw
// (before BCNorm and rotation), as m3_layer_prefill takes them.
struct BackwardArgs {
    const void* x;
    const void* B;
    const void* C;
    const void* dt;
    const void* theta;
    const float* A;
    const void* lam;
    const float* normw_B;
    const float* normw_C;
    const float* bias_B;
    const float* bias_C;
    const float* w_out;
    const float* phi_in;
    const float* h_in;
    const void* Bbar_prev;
    const void* x_prev;
    // cotangents of y, h_out, phi_out (the last two nullable: zero)
    const void* dy;
    const float* dh_out;
    const float* dphi_out;
    // gradients
    void* dx;
    void* dB;
    void* dC;
    void* ddt;
    void* dtheta;
    void* dlam;
    float* dA;
    float* dnormw_B;
    float* dnormw_C;
    float* dbias_B;
    float* dbias_C;
    float* dw_out;
    float* dphi_in;
    float* dh_in;
    void* dBbar_prev;
    void* dx_prev;
    // workspace: chunk-entry states [b, H, nchunk, P, N] (io type), entry angles
    // [b, H, nchunk, N/2], per-(b, h) partial sums [b, H, rec], per-chunk step sums and dA share
    // [b, H, nchunk, 5 Q + 3] (f32; see step_grads_kernel)
    void* ws_states;
    float* ws_phi;
    float* ws_part;
    float* ws_scal;
    int rec;              // 1 + R P + 2 N + 2 R N
    int64_t b, L;
    int H, N, P, R;
    int bcnorm;
    float eps;
    // raw B and C hold G head slots, head h reads slot h / (H / G) (0: one slot per head).  With
    // G < H the backward kernel writes each head's dB, dC rows to ws_dB, ws_dC ([b, L, H, R, N]
    // io) and group_sum adds each group's heads into dB, dC.
    int G = 0;
    void* ws_dB = nullptr;
    void* ws_dC = nullptr;
};

bool backward_supported(int N, int P, int R);
int backward_chunk_rows(int P, bool bf16_io);   // rows (step, rank) per chunk; steps = rows / R
hipError_t launch_chunk_states(const BackwardArgs& a, bool bf16_io, hipStream_t s);
hipError_t launch_backward(const BackwardArgs& a, bool bf16_io, hipStream_t s);

bool decode_supported(int N, int P, int R);
hipError_t launch_decode(const DecodeArgs& a, bool bf16_io, hipStream_t s);
hipError_t launch_layer_decode(const DecodeArgs& a, bool bf16_io, hipStream_t s);

bool bcnorm_rope_supported(int N, int R);
int64_t bcnorm_rope_seglen();
int bcnorm_rope_parts();   // quarters per segment: the workspace holds one angle row per quarter
hipError_t launch_bcnorm_rope(const BcnormRopeArgs& a, bool bf16_io, hipStream_t s);

bool prefill_supported(int N, int P, int R, int QR, bool bf16_io);
hipError_t launch_prefill(const PrefillArgs& a, bool bf16_io, hipStream_t s);

bool layer_supported(int N, int P, int R, int QR, bool bf16_io);
hipError_t launch_layer(const PrefillArgs& a, bool bf16_io, hipStream_t s);
// between the two passes of a split sequence: true start angles, end states and last Bbar rows
hipError_t launch_segment_combine(const PrefillArgs& a, bool bf16_io, hipStream_t s);

}  // namespace m3
