/*
 * CPU oracle for the MXFP4 routed-expert MoE layer -- TEST INFRASTRUCTURE.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this.  The GPU library shares no code, header, table or helper
 * with it; the two meet only through the seeded input generator.
 *
 * Every function computes the plain definition, slowly and in the order the
 * definition states.  Page citations name the page title and its section.
 *
 * Layouts (all canonical, row-major, little-endian):
 *   MXFP4 matrix with R rows and K columns:
 *     codes  uint8 [R][K/2]   element k of a row sits in byte k/2,
 *                              low nibble for even k, high nibble for odd k
 *     scales uint8 [R][K/32]  one UE8M0 byte per 32 consecutive elements
 *   w13: [E_local][2I][H] (rows 0..I-1 = gate, rows I..2I-1 = up)
 *   w2 : [E_local][H][I]
 *   x  : bf16 bits [T][H];  router logits: float [T][E_global]
 *   out: float [T][H] before rounding (out32) and bf16 bits [T][H]
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t T, H, I;
  int64_t E_global, E_local, first_local;
  int32_t top_k;
  float clamp_limit;
  int32_t a4; /* 1: x and the SwiGLU output are MXFP4-quantised before each contraction */
  int32_t shared; /* 1: the weight buffers hold E_local + 1 experts; the last is a shared
                     expert every token reads with weight 1 (slot k of each token) */
  int32_t given_actq; /* A4/A8 only, 1: down reads actq/acts as inputs (the quantised SwiGLU
                         output of another implementation, rows in sorted order)
                         instead of quantising its own; everything else unchanged */
  int32_t a8; /* 1: as a4 with MXFP8 (E4M3 elements, one byte each): xq [T][H],
                 actq [N][I]; scales as for a4.  a4 and a8 exclude each other */
  /* Per-expert exclusions (nullable): bf16_expert[e] != 0 marks expert e of the
   * weight buffers as stored in bf16 instead of MXFP4.  Its weights are then
   * read from w13_bf16 [n][2I][H] and w2_bf16 [n][H][I] (bf16 bits; slot j is
   * the j-th excluded expert in expert order) and its slots in w13/w13s/w2/w2s
   * are ignored.  Such an expert computes on the bf16 x and the bf16 SwiGLU
   * output in every activation mode (no A4/A8 quantisation; its actq/acts rows
   * are left untouched). */
  const uint8_t* bf16_expert;
  const uint16_t* w13_bf16;
  const uint16_t* w2_bf16;
} orc_dims;

/* element and scale decoding */
double orc_e2m1_value(int32_t code);
double orc_ue8m0_value(int32_t s);
void orc_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                 float* out);

/* OCP MX quantiser, one 32-element block at a time along each row */
void orc_quantize_f64(const double* v, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales);
void orc_quantize_f32(const float* v, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales);
void orc_quantize_bf16(const uint16_t* v, int64_t rows, int64_t K, uint8_t* codes,
                       uint8_t* scales);

/* MXFP8: E4M3 element value (0x7F/0xFF NaN), quantiser (codes one byte per
 * element, [rows][K]; scales [rows][K/32]) and dequantiser */
double orc_e4m3_value(int32_t code);
void orc_quantize8_bf16(const uint16_t* v, int64_t rows, int64_t K, uint8_t* codes,
                        uint8_t* scales);
void orc_quantize8_f64(const double* v, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales);
void orc_dequant8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                  float* out);

/* fp32 -> bf16, round to nearest even */
uint16_t orc_bf16_from_f32(float f);
void orc_bf16_round_array(const float* in, int64_t n, uint16_t* out);
float orc_f32_from_bf16(uint16_t b);

/* router: softmax over all global experts, top-k, renormalise over the k picks */
int orc_route(const float* logits, int64_t T, int64_t E_global, int32_t k, int32_t* ids, float* w);

/* local filter + histogram + exclusive scan + stable scatter; returns N_assign.
 * shared_id >= 0: slots with that id go to table entry E_local (the shared
 * expert; counts/offsets then have E_local + 1 / E_local + 2 entries). */
int64_t orc_permute(const int32_t* ids, int64_t T, int32_t k, int64_t first_local, int64_t E_local,
                    int64_t shared_id, int32_t* counts, int32_t* offsets, int32_t* sorted,
                    int32_t* inv);

/* clamped SwiGLU of one (gate, up) pair in fp32 */
float orc_swiglu(float g, float u, float limit);

/*
 * Full layer.  token_mask (nullable, uint8 [T]) restricts the expert work and
 * the combine to the tokens whose mask byte is non-zero; the routing tables are
 * always produced for every token.  Outputs that are NULL are not written.
 *   (with the shared expert read k as top_k + 1 and E_local as E_local + 1 below;
 *    ids[t][top_k] = E_global and w[t][top_k] = 1 mark the shared slot)
 *   ids/w      [T][k]             counts [E_local], offsets [E_local+1]
 *   sorted/inv [T*k]              act bf16 bits [T*k][I] (row p = sorted position p)
 *   xq/xs      [T][H/2], [T][H/32]          (A4 only)
 *   actq/acts  [T*k][I/2], [T*k][I/32]      (A4 only)
 *   out32 float [T][H], out bf16 bits [T][H]
 * Returns N_assign (>= 0) or a negative value on bad arguments.
 */
int64_t orc_moe_forward(const orc_dims* d, const uint16_t* x, const float* logits,
                        const uint8_t* w13, const uint8_t* w13s, const uint8_t* w2,
                        const uint8_t* w2s, const uint8_t* token_mask, int32_t* ids, float* w,
                        int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* inv,
                        uint16_t* act, uint8_t* xq, uint8_t* xs, uint8_t* actq, uint8_t* acts,
                        float* out32, uint16_t* out, int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
