"""The store's token-span allocator (kv_cache_injection_is_amd/csrc/arena.h,
used by is_store_append and is_store_remove) against a brute-force model of
every arena token, over random allocate/free sequences: first-fit
placement, freed spans merged with their neighbours, the end of the used
arena moving back, no token handed out twice, and all-or-nothing refusal
when nothing fits.  Host code only: compiled here with g++."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "kv_cache_injection_is_amd", "csrc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("arena") / "arena_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", CSRC,
                    os.path.join(HERE, "arena_check.cpp"), "-o", exe], check=True)
    return exe


@pytest.mark.parametrize("seed", range(12))
def test_arena_matches_the_token_model(checker, seed):
    r = subprocess.run([checker, str(seed), "3000"], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
