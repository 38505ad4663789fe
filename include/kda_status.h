/*
 * kda_status.h -- return codes and limits of the KDA library's C ABI
 * (include/kda.h).  Kept apart from kda.h, which needs the HIP runtime
 * headers for hipStream_t, so that host-only code (the argument checks built
 * with a plain C++ compiler) can use the same definitions.
 */
#ifndef KDA_STATUS_H_
#define KDA_STATUS_H_

/* Return codes of kda_chunk_fwd (0 = success). */
enum kda_status {
  KDA_OK = 0,
  KDA_ERR_NULL_PTR = -1,    /* a required pointer is NULL                              */
  KDA_ERR_BAD_SHAPE = -2,   /* T < 0, T > INT32_MAX, H < 1 or H > KDA_MAX_HEADS         */
  KDA_ERR_UNSUPPORTED = -3, /* chunk != 64, or gate_bound not finite or outside [-5.5, 0) */
  KDA_ERR_ALIGN = -4,       /* q, k, v, g, out not 16-byte aligned; beta, cu_seqlens not 4-byte aligned */
  KDA_ERR_HIP = -5,         /* a HIP runtime call or kernel launch failed              */
  KDA_ERR_ALLOC = -6        /* the stream-ordered workspace allocation failed          */
};

/* Bits of the sticky device status word (kda_device_status). */
enum kda_device_flags {
  KDA_DEV_BAD_CU_SEQLENS = 1, /* cu_seqlens broke its contract; out was filled with NaN  */
  KDA_DEV_GATE_RANGE = 2      /* some g fell outside [gate_bound, 0] (or was NaN); the
                                 result was still computed, without clamping             */
};

#define KDA_HEAD_DIM 128
#define KDA_CHUNK 64
#define KDA_MAX_HEADS 4096

#endif /* KDA_STATUS_H_ */
