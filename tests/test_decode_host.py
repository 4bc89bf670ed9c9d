"""The library's bit-plane network, run on the CPU, against the oracle.

tests/native/decode_harness.hip compiles decode.h -- the very functions the
kernels inline -- for the host and applies them with the kernels' chunk
indexing.  This checks the packer network, the unpack network, the bf16
operand decode (magic exponents, offsets, coefficients) and the single-phase
byte decode of the large-batch GEMM bit for bit without a GPU.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from nested_bit_weight_amd import build as nbw_build

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("harness") / "decode_harness")
    cmd = [nbw_build.hipcc(), *nbw_build.compile_flags(), os.path.join(HERE, "native",
                                                                        "decode_harness.hip"),
           "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return out


def _run(harness, mode, n, k, r, data, tmp_path):
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    fin.write_bytes(np.ascontiguousarray(data).tobytes())
    subprocess.run([harness, mode, str(n), str(k), str(r), str(fin), str(fout)], check=True)
    return fout.read_bytes()


def test_pack_network_matches_oracle(harness, tmp_path):
    n, k = 37, 640
    codes = synth.uniform_codes(n, k, np.random.default_rng(21))
    got = np.frombuffer(_run(harness, "pack", n, k, 8, codes, tmp_path), dtype=np.uint8)
    np.testing.assert_array_equal(got, oracle.pack(codes))


@pytest.mark.parametrize("r", range(1, 9))
def test_unpack_network_matches_oracle(harness, tmp_path, r):
    n, k = 21, 384
    i = np.arange(n)[:, None]
    j = np.arange(k)[None, :]
    codes = ((i * 3 + j * 5) % 256).astype(np.uint8)
    planes = oracle.pack(codes)
    got = np.frombuffer(_run(harness, "unpack", n, k, r, planes, tmp_path), dtype=np.uint8)
    np.testing.assert_array_equal(got.reshape(n, k), oracle.unpack(planes, n, k, r))


@pytest.mark.parametrize("r", range(1, 9))
def test_bf16_operands_decode_to_codes(harness, tmp_path, r):
    # decoded bf16 operand minus its constant offset must equal the child code
    n, k = 19, 256
    codes = synth.uniform_codes(n, k, np.random.default_rng(22 + r))
    planes = oracle.pack(codes)
    got = np.frombuffer(_run(harness, "operands", n, k, r, planes, tmp_path), dtype=np.float32)
    np.testing.assert_array_equal(got.reshape(n, k), oracle.unpack(planes, n, k, r).astype(np.float32))


@pytest.mark.parametrize("r", range(5, 9))
def test_byte_operands_decode_to_codes(harness, tmp_path, r):
    # the single-phase bf16 operand is the child code times 2^(8-r), exactly
    n, k = 19, 384
    codes = synth.uniform_codes(n, k, np.random.default_rng(40 + r))
    planes = oracle.pack(codes)
    got = np.frombuffer(_run(harness, "bytes", n, k, r, planes, tmp_path), dtype=np.float32)
    np.testing.assert_array_equal(got.reshape(n, k), oracle.unpack(planes, n, k, r).astype(np.float32))
