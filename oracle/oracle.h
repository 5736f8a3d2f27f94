/* CPU oracle for MoE dispatch / combine -- test infrastructure only.
 * Declarations for oracle.c; nothing outside oracle/ includes this file. */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

enum { ORACLE_OK = 0, ORACLE_INVALID_ARG = 1, ORACLE_UNSUPPORTED = 2, ORACLE_BAD_EXPERT_ID = 3 };

int oracle_check_shape(int64_t T, int64_t H, int32_t E, int32_t k, int32_t R, int32_t C, int fp8);
int oracle_layout(int64_t T, int32_t E, int32_t k, int32_t R, int32_t C, const int32_t *topk_idx,
                  int32_t *pos, int32_t *expert_count, int32_t *rank_count, int32_t *recv_offset,
                  int32_t *send_offset, int32_t *chunk_offset, int32_t *recv_src);
int oracle_layout_grouped(int64_t T, int32_t E, int32_t k, int32_t R, int32_t C,
                          const int32_t *topk_idx, int32_t *pos, int32_t *expert_count,
                          int32_t *expert_offset, int32_t *rank_count, int32_t *recv_offset,
                          int32_t *send_offset, int32_t *chunk_offset, int32_t *recv_src);
float oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f32_to_bf16(float f);
float oracle_e4m3_to_f32(uint8_t c);
uint8_t oracle_f32_to_e4m3(float f);
void oracle_dispatch_bf16(int64_t T, int64_t H, int32_t k, const uint16_t *x, const int32_t *pos,
                          uint16_t *recv);
void oracle_dispatch_fp8(int64_t T, int64_t H, int32_t k, const uint16_t *x, const int32_t *pos,
                         uint8_t *recv8, float *recv_scale);
void oracle_identity_fp8(int64_t rows, int64_t H, const uint8_t *q, const float *scale,
                         uint16_t *y);
void oracle_combine(int64_t T, int64_t H, int32_t k, const uint16_t *y, const int32_t *pos,
                    const float *topk_w, uint16_t *out);
void oracle_f32_to_e4m3_array(int64_t n, const float *in, uint8_t *out);
void oracle_f32_to_bf16_array(int64_t n, const float *in, uint16_t *out);
void oracle_e4m3_to_f32_array(int64_t n, const uint8_t *in, float *out);
enum { ORACLE_GATE_SOFTMAX = 0, ORACLE_GATE_SIGMOID = 1 };
int oracle_gate(int64_t T, int32_t E, int32_t k, int32_t groups, int32_t keep_groups, int norm,
                const float *logits, int32_t *topk_idx, float *topk_w);

uint16_t oracle_f64_to_bf16(double v);
void oracle_expert_linear(int32_t E, int64_t H, int64_t N, const int32_t *expert_offset,
                          const uint16_t *x, const uint16_t *w, uint16_t *y);

#endif
