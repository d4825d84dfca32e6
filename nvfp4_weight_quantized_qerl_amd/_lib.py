"""ctypes declarations of libqerl.so (the C ABI in include/qerl.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any call.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqerl.so")

c_i32, c_i64, c_u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
c_f32, c_f64, c_sz, c_vp = ctypes.c_float, ctypes.c_double, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes); the order follows include/qerl.h
SIGNATURES = {
    "qerl_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "qerl_abi_version": (ctypes.c_int, []),
    "qerl_quantize_nvfp4": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "qerl_quantize_nvfp4_batch": (ctypes.c_int, [c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                 c_vp]),
    "qerl_quantize_mxfp4": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "qerl_mxfp4_to_nvfp4": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp]),
    "qerl_nvfp4_check_pow2_scales": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_vp]),
    "qerl_aqn_sigma": (ctypes.c_int, [c_f64, c_f64, c_i32, c_i32, ctypes.POINTER(c_f64)]),
    "qerl_aqn_sigma_schedule": (ctypes.c_int, [c_i32, c_f64, c_f64, c_i32, c_i32,
                                                ctypes.POINTER(c_f64)]),
    "qerl_aqn_sample": (ctypes.c_int, [c_u64, c_u64, c_u64, c_f64, c_i64, c_vp, c_vp]),
    "qerl_aqn_sample_batch": (ctypes.c_int, [c_u64, c_u64, c_u64, c_u64, c_i64, c_f64, c_i64,
                                             c_vp, c_vp]),
    "qerl_aqn_sample_rows": (ctypes.c_int, [c_u64, c_u64, c_u64, c_f64, c_i64, c_i64, c_vp,
                                            c_vp]),
    "qerl_linear_decode_rownoise": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                   c_vp, c_vp, c_i32, c_f32, c_vp, c_vp, c_vp,
                                                   c_sz, c_vp]),
    "qerl_linear_prefill_rownoise": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                    c_vp, c_vp, c_i32, c_f32, c_vp, c_vp, c_vp,
                                                    c_sz, c_vp]),
    "qerl_attention_stub": (ctypes.c_int, [c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "qerl_rmsnorm_noisy": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_vp, c_f32, c_vp, c_vp]),
    "qerl_swiglu": (ctypes.c_int, [c_vp, c_i64, c_i64, c_vp, c_vp]),
    "qerl_linear_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i32]),
    "qerl_linear_decode": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64, c_vp,
                                          c_vp, c_i32, c_f32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "qerl_linear_decode_swiglu": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                 c_vp, c_vp, c_i32, c_f32, c_vp, c_vp, c_vp,
                                                 c_sz, c_vp]),
    "qerl_linear_prefill": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64, c_vp,
                                           c_vp, c_i32, c_f32, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "qerl_linear_prepare": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i32, c_f32,
                                           c_vp, c_vp, c_sz, c_vp]),
    "qerl_linear_decode_prepared": (ctypes.c_int, [c_i64, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                   c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]),
    "qerl_linear_prefill_prepared": (ctypes.c_int, [c_i64, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                    c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]),
    "qerl_linear_decode_mxfp4": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                c_vp, c_vp, c_i32, c_f32, c_vp, c_vp, c_vp, c_sz,
                                                c_vp]),
    "qerl_linear_decode_prepared_mxfp4": (ctypes.c_int, [c_i64, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                         c_vp, c_i32, c_vp, c_vp, c_sz, c_vp]),
    "qerl_nvfp4_tile128_bytes": (c_sz, [c_i64, c_i64]),
    "qerl_nvfp4_tile128": (ctypes.c_int, [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp]),
    "qerl_linear_tiled_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i32]),
    "qerl_linear_decode_tiled": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp, c_i64, c_i64, c_vp,
                                                c_vp, c_i32, c_f32, c_vp, c_vp, c_vp, c_sz,
                                                c_vp]),
    "qerl_linear_decode_tiled_prepared": (ctypes.c_int, [c_i64, c_vp, c_vp, c_i64, c_i64, c_vp,
                                                         c_i32, c_vp, c_vp, c_sz, c_vp]),
    "qerl_linear_noalloc_scratch_bytes": (c_sz, []),
    "qerl_linear_decode_noalloc": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64,
                                                  c_vp, c_vp, c_i32, c_f32, c_vp, c_vp, c_vp]),
    "qerl_linear_backward_workspace_bytes": (c_sz, [c_i64, c_i64, c_i64, c_i32]),
    "qerl_linear_backward": (ctypes.c_int, [c_vp, c_i64, c_vp, c_vp, c_vp, c_i64, c_i64, c_vp,
                                            c_vp, c_vp, c_i32, c_f32, c_vp, c_vp, c_vp, c_vp,
                                            c_vp, c_sz, c_vp]),
}


def load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python nvfp4_weight_quantized_qerl_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib
