// Shared declarations of the HIP kernels' parameter blocks and launchers.
// Device code targets gfx950 (CDNA4, wave64) only.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace sv {

// ---------------------------------------------------------------- tiling
// A weight "fragment" is the B operand of one v_mfma_f32_16x16x32_bf16:
// 16 output columns x 32 k.  Lane l holds 8 consecutive k of column l%16:
// k = 8*(l/16) + e, e = 0..7 (16 bytes, bf16).  Fragments of one 16-column
// tile ("n-tile") are contiguous along k, so a wave streams a tile's K
// extent as consecutive 1 KB blocks.
constexpr int kWave = 64;
constexpr int kTileN = 16;
constexpr int kChunkK = 32;
constexpr int kGroupK = 128;          // int4 scale group along K
constexpr int kWavesPerWG = 4;
constexpr int kColsPerWG = kWavesPerWG * kTileN;   // 64 output columns / WG
constexpr int kMaxRows = 16;          // block rows (k+1) per pass
constexpr int kPage = 64;             // KV page = attention chunk (positions)

enum WFmt : int { W_BF16 = 0, W_INT4 = 1, W_F32 = 2 };
enum Epi : int { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

struct GemmParams {
  int m;              // live rows (<= 16)
  int K;              // logical K
  int nkc;            // K chunks of 32 in the fragment layout (padded)
  int N;              // logical output columns (SWIGLU: act columns)
  int n_tiles;        // weight n-tiles (SWIGLU: 2 per act tile, interleaved gate/up)
  int kcs;            // chunks per split-K slice
  int splits;         // number of K slices
  // activations
  const float* x; int ldx; long long x_stride;   // x_stride: per expert slot (MoE down)
  const float* ss; int n_ss; float inv_dnorm; float eps;   // RMSNorm prologue (ss == nullptr: none)
  const float* gain;                                      // per-k gain (nullptr: 1)
  // weights
  const void* w;            // fragments (bf16 / int4) or hi fragments (f32)
  const void* w2;           // lo fragments (f32) or fp16 scales (int4)
  long long w_stride;       // bytes between experts (MoE)
  long long w2_stride;
  // split-K scratch
  float* ws; unsigned* counters;
  // outputs
  float* out; int ldo; long long out_stride;   // per expert slot (MoE)
  float* ss_out; int n_ss_out;                 // RESID: sum-of-squares partials of new x
  float* st_max; float* st_sum; int* st_idx; int n_stat;   // LOGITS partials (per 64 cols)
  // MoE expert dispatch (nullptr: dense)
  const int* union_count; const int* union_list; int n_experts; int n_shared;
};

struct AttnParams {
  int m, L, G;           // block rows, committed length, query heads per KV head
  int Hq, Hkv, D;
  int n_chunks;
  const float* qkv; int ldqkv;     // [m][(Hq+2Hkv)*D]
  const float* rope_cs;            // [max_ctx][D/2][2] (cos, sin)
  void* kv;                        // layer base: pages [page][Hkv][2][kPage][D]
  const int* page_table;
  float* pm; float* ps; float* pacc;   // partials [Hkv][n_chunks][R] / [..][R][D]
  int R;                           // m*G
  float scale;                     // 1/sqrt(D)
};

struct CombineParams {
  int m, G, Hq, D, n_chunks, R;
  const float* pm; const float* ps; const float* pacc;
  float* o; int ldo;
};

struct AcceptParams {
  int k, V, L, mode, n_stat;
  const int* tokens;
  const float* st_max; const float* st_sum; const int* st_idx;
  const float* logits; int ldl;
  const float* q; const float* u;
  int* result;          // [3]
};

struct RouteParams {
  int m, E, top_k;
  const float* rlogits; int ldr;   // [m][E] router logits (without bias)
  const float* bias;
  int* union_count; int* union_list; int* sel; float* selw; int* slot_of;
  int* union_hist;       // nullable: per-layer |U| record
};

struct MoeCombineParams {
  int m, d, top_k, n_shared, n_ss;
  const int* union_count; const int* sel; const float* selw; const int* slot_of;
  const float* y; long long y_stride; int ldy;   // [slot][m][d]
  float* x; int ldx; float* ss_out;
};

// ---------------------------------------------------------------- launchers
hipError_t launch_gemm(int wfmt, int epi, const GemmParams& p, int n_slots, hipStream_t s);
hipError_t launch_attention(int kv_f32, const AttnParams& p, hipStream_t s);
hipError_t launch_attn_combine(const CombineParams& p, hipStream_t s);
hipError_t launch_embed(int emb_f32, const void* table, const int* tokens, int m, int d,
                        float* x, float* ss_out, hipStream_t s);
hipError_t launch_route(const RouteParams& p, hipStream_t s);
hipError_t launch_moe_combine(const MoeCombineParams& p, hipStream_t s);
hipError_t launch_accept(const AcceptParams& p, hipStream_t s);
hipError_t launch_retile_bf16(const uint16_t* src, int K, int N, void* dst, int nkc,
                              int tile_off, int tile_stride, hipStream_t s);
hipError_t launch_retile_f32(const float* src, int K, int N, void* dst_hi, void* dst_lo, int nkc,
                             int tile_off, int tile_stride, hipStream_t s);
hipError_t launch_retile_int4(const uint8_t* src_q, const uint16_t* src_s, int K, int N, void* dst,
                              void* dst_s, int tile_off, int tile_stride, int n_tiles_total,
                              hipStream_t s);
hipError_t launch_kv_import(int kv_f32, const void* src, int P, int Hkv, int D, void* layer_base,
                            const int* page_table, hipStream_t s);

}  // namespace sv
