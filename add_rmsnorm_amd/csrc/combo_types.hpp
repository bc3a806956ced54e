// The (row dtype, weight dtype) pair of one compilation of tables.hip or
// rope.hip, from ADDRMS_COMBO = 3 * row_dtype + weight_dtype with the dtype
// codes of addrms.h (0 = float32, 1 = bfloat16, 2 = float16).  The build
// compiles each file once per combination so the instantiations compile in
// parallel.
#pragma once

#ifndef ADDRMS_COMBO
#error "define ADDRMS_COMBO (0..8)"
#endif

#if ADDRMS_COMBO / 3 == 0
#define ADDRMS_ROW_T float
#elif ADDRMS_COMBO / 3 == 1
#define ADDRMS_ROW_T addrms::bf16_t
#elif ADDRMS_COMBO / 3 == 2
#define ADDRMS_ROW_T addrms::f16_t
#else
#error "ADDRMS_COMBO out of range (0..8)"
#endif

#if ADDRMS_COMBO % 3 == 0
#define ADDRMS_W_T float
#elif ADDRMS_COMBO % 3 == 1
#define ADDRMS_W_T addrms::bf16_t
#else
#define ADDRMS_W_T addrms::f16_t
#endif

#define ADDRMS_CAT2(a, b) a##b
#define ADDRMS_CAT(a, b) ADDRMS_CAT2(a, b)
